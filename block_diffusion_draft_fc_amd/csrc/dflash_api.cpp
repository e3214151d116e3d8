// C ABI of the DFlash KV-injection attention library: argument validation,
// host-side cache metadata, work planning and the launch sequence of each call.
// Every check runs before the first enqueue, so a call that fails validation
// changes no state.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <vector>

#include "dflash.h"
#include "kernels.hpp"

using namespace dflash;

struct dflash_cache {
  dflash_cache_desc desc;
  std::vector<int32_t> len;
  std::vector<int64_t> written_hi;          // ring: highest position ever written + 1
  std::vector<std::vector<int32_t>> pages;   // paged: physical page per logical page
  std::set<int32_t> free_pages;             // paged: lowest first
  // device-driven rounds: the true lengths live in d_len on the device; len
  // then holds upper bounds of them (every round counted with its largest
  // possible number of new rows), and the pages cover the bounds
  int32_t* d_len = nullptr;
  bool dev = false;
};

namespace {

constexpr size_t kAlign = 256;
// Upper bound on attention work items per call beyond one per (sequence, head).
constexpr int kAttnMaxTarget = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool dtype_ok(int32_t dt) { return dt == DFLASH_F32 || dt == DFLASH_BF16; }
bool cache_dtype_ok(int32_t dt) { return dtype_ok(dt) || dt == DFLASH_FP8_E4M3; }
bool scale_ok(float x) { return std::isfinite(x) && x > 0.f; }
size_t elem_bytes(int32_t dt) { return dt == DFLASH_BF16 ? 2 : 4; }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- stage timing
// While enabled, each stage of a call is bracketed by two HIP events recorded
// on the caller's stream; the elapsed times are collected when read.
struct TimingRec {
  int stage;
  hipEvent_t a, b;
};
struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<TimingRec> pending;
  int64_t launches[DFLASH_STAGE_COUNT] = {};
  double ms[DFLASH_STAGE_COUNT] = {};
};
Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t take_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace dflash {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace dflash

namespace {

// Runs `f` (which enqueues the stage's kernels on `s`).  With timing on, the
// stage's kernels carry an event pair (hipExtLaunchKernel start/stop events,
// stamped when the kernels themselves start and end on the GPU); a stage that
// launched nothing records nothing.
// Calls that must not create events (the scratch-buffer entry point) run
// their stages without timing.
thread_local bool t_untimed = false;

template <class F>
hipError_t staged(int stage, hipStream_t s, bool launches, F&& f) {
  (void)s;
  Timing& t = timing();
  if (!launches || t_untimed) return f();
  bool on;
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> g(t.mu);
    on = t.on;
    if (on) {
      a = take_event(t);
      b = take_event(t);
    }
  }
  if (!on || !a || !b) return f();
  LaunchEvents& ev = launch_events();
  ev.start = a;
  ev.stop = b;
  const hipError_t e = f();
  const bool launched = ev.start == nullptr;
  ev.start = nullptr;
  ev.stop = nullptr;
  std::lock_guard<std::mutex> g(t.mu);
  if (e == hipSuccess && launched) {
    t.pending.push_back({stage, a, b});
  } else {
    t.pool.push_back(a);
    t.pool.push_back(b);
  }
  return e;
}

// How one attention launch splits the keys into work items (sequence, K/V
// head, chunk of `chunk` keys) and which ring depth runs them.
//  * Ring depth: up to 256K keys over all (sequence, K/V head) pairs, three
//    stages and one workgroup per CU (the 8K decode round: each CU's ring
//    runs two blocks ahead of its compute); beyond, two stages and two
//    workgroups per CU, which cover each other's load latency.
//  * Item count: the CUs hold `slots` workgroups at once (256 or 512).  Items
//    past a whole round of slots would run by themselves at the end (a few
//    items over 512 cost a third of the time on the 16-request ragged batch),
//    so the chunk is the smallest multiple of 64 keys (at least 128) whose
//    items fit one round.  Two rounds balanced the unequal last chunks of the
//    ragged batch and the 5-layer stack no better than they cost in partials.
// dflash_attn_force_chunk replaces the chunk (a diagnostic: the result must
// not depend on the split).
struct AttnSplit {
  int64_t chunk;
  int64_t items;
  int nst;
};

std::atomic<int64_t> g_forced_chunk{0};
std::atomic<int> g_merge_spread{0};   // dflash_attn_force_merge_spread
std::atomic<int> g_spin_limit{kAttnSpinLimit};   // dflash_attn_set_spin_limit

AttnSplit plan_attn_split(const std::vector<int64_t>& keys, int n_kv, int64_t chunk_cap, bool fp8) {
  int64_t total = 0;
  for (int64_t k : keys) total += k * n_kv;
  AttnSplit sp{};
  sp.nst = total > ((int64_t)256 << 10) ? 2 : 3;
  auto items_of = [&](int64_t chunk) {
    int64_t it = 0;
    for (int64_t k : keys) it += std::max<int64_t>(1, cdiv(k, chunk)) * n_kv;
    return it;
  };
  const int64_t cap = std::max<int64_t>(128, chunk_cap / 64 * 64);
  const int64_t forced = g_forced_chunk.load();
  if (forced > 0) {
    sp.chunk = std::min(cap, forced);
  } else {
    // workgroup slots of one round: 256 at depth 3 (one per CU), 512 at depth
    // 2 (two per CU); fp8 caches at depth 2 fit four per CU (32 KB of LDS and
    // at most 128 VGPRs each): 4 x 32K keys 79 us with two per CU, 73 with
    // three, 67 with four
    const int64_t slots = sp.nst == 2 ? (fp8 ? 1024 : 512) : 256;
    const int64_t limit = std::min<int64_t>(kAttnMaxTarget, slots);
    // items_of is non-increasing in the chunk: the smallest chunk (in units of
    // 64 keys) in [2, cap / 64] with items_of <= limit, else the cap
    int64_t lo = 2, hi = cap / 64;
    if (items_of(hi * 64) > limit) {
      lo = hi;
    } else {
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (items_of(mid * 64) <= limit) hi = mid; else lo = mid + 1;
      }
    }
    sp.chunk = lo * 64;
  }
  sp.items = items_of(sp.chunk);
  return sp;
}

// ---------------------------------------------------------------- GEMM planning

struct SkinnyPlan {
  int32_t k_chunk, splits, mt, n_tiles;
  bool wide;         // gemm_wide_kernel (256-column tiles) instead of gemm_lds_kernel
  bool tile;         // gemm_tile_kernel (256x256 MFMA tiles) for many rows
  bool stream;       // gemm_stream_kernel (per-wave weight streams) for at most 64 rows
  bool fullk;        // gemm_fullk_kernel (no split-K partials) for at most 16 rows
  bool resident;     // gemm_resident_kernel: at most 16 rows kept in LDS, very many columns
  bool slab;         // gemm_slab_kernel: bf16, up to 128 rows, slice staged in up to 160 KB of LDS
  int32_t m_tiles;   // tile plans only
  int32_t tile_bn;   // tile plans only: output columns per tile
};


// Whether a product may take gemm_slab_kernel: bf16 and K a multiple of 512.
bool slab_eligible(int64_t K, size_t eb) { return eb == 2 && K % 512 == 0; }

// Rows per weight-streaming problem: 128 for slab-eligible products with K
// up to 8192 (the kernel's row limit), else
// 64 for bf16 and 32 for fp32, whose staged activation rows take twice the
// LDS (this keeps every gemm_lds_kernel plan within its 64 KB dynamic LDS
// budget).  Above 64 rows the slab kernel's chunk is 512 wide, so its fp32
// partials weigh half the weights: fine for a 4096-wide input (the 5-layer
// stack's K/V product beats the tile kernel), not for the 20480-wide fc,
// where the tile kernel takes 65+ rows (ragged batch fc: 64 -> 47 us).
int64_t rows_per_problem(int64_t K, size_t eb) {
  if (slab_eligible(K, eb)) return K <= 8192 ? 128 : kSkinnyMaxM;
  return eb == 2 ? kSkinnyMaxM : kSkinnyMaxM / 2;
}

// Plans for at most 128 rows (64 or 32 without the slab kernel), tuned on the
// decode-round shapes:
//  * long inputs (K >= 8192, bf16, <= 32 rows): gemm_wide_kernel, 256-column
//    tiles, about 256 workgroups with chunks of whole 128-wide stages;
//  * otherwise gemm_lds_kernel, 64-column tiles, about 1024 workgroups with
//    256-wide chunks, the staged activation slice within the LDS budget.
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, size_t eb) {
  constexpr int wide_target = 256, lds_target = 1024, wide_min_k = 8192;
  SkinnyPlan p{};
  p.mt = (int32_t)std::max<int64_t>(1, cdiv(M, 16));
  // at most 16 rows and very many columns (a vocabulary): the rows stay in
  // LDS and each wave streams whole weight tiles, one result
  if (eb == 2 && p.mt == 1 && K % 64 == 0 && K <= kResMaxK && N % 4 == 0 && N >= 65536) {
    p.resident = true;
    p.n_tiles = (int32_t)cdiv(N, 16);
    p.k_chunk = (int32_t)K;
    p.splits = 1;
    return p;
  }
  // at most 16 rows: the whole K in one workgroup per 16 columns, one result
  if (eb == 2 && p.mt == 1 && K % 512 == 0 && N % 4 == 0) {
    p.fullk = true;
    p.n_tiles = (int32_t)cdiv(N, 16);
    p.k_chunk = (int32_t)K;
    p.splits = 1;
    return p;
  }
  // at most 64 rows, K below the wide kernel's range: per-wave weight streams
  // in 512-wide K-chunks
  if (eb == 2 && p.mt <= 4 && K < wide_min_k && K % 64 == 0 && N % 4 == 0) {
    p.stream = true;
    p.n_tiles = (int32_t)cdiv(N, 16 * gemm_stream_waves(p.mt));
    p.k_chunk = 512;
    p.splits = (int32_t)cdiv(K, 512);
    return p;
  }
  // 65..128 rows, or 33..64 with a long K (bf16, K a multiple of 512): the
  // slice staged by direct copies in up to 160 KB of LDS, which allows
  // 1024-wide chunks at 64 rows and 512-wide at 128; splits to about one
  // workgroup per CU
  if (slab_eligible(K, eb) && p.mt >= 3 && p.mt <= 8) {
    constexpr int slab_target = 256;
    p.slab = true;
    p.n_tiles = (int32_t)cdiv(N, 64);
    const int64_t kmax = std::max<int64_t>(512, ((int64_t)kSlabLdsBytes / (p.mt * 16 * 2) - 8) / 512 * 512);
    int64_t splits = std::max<int64_t>(cdiv(K, kmax), cdiv(slab_target, p.n_tiles));
    splits = std::min<int64_t>(splits, K / 512);
    const int64_t kc = cdiv(cdiv(K, splits), 512) * 512;
    p.k_chunk = (int32_t)kc;
    p.splits = (int32_t)cdiv(K, kc);
    return p;
  }
  p.wide = eb == 2 && p.mt <= 2 && K >= wide_min_k;
  if (p.wide) {
    p.n_tiles = (int32_t)cdiv(N, 256);
    int64_t splits = std::max<int64_t>(1, cdiv(wide_target, p.n_tiles));
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, cdiv(K, 128)));
    const int64_t kc = cdiv(cdiv(K, splits), 128) * 128;
    p.k_chunk = (int32_t)kc;
    p.splits = (int32_t)cdiv(K, kc);
    return p;
  }
  p.n_tiles = (int32_t)cdiv(N, 64);
  int64_t kmax = ((int64_t)kLdsGemmBytes / (int64_t)(p.mt * 16 * eb) - 8) / 256 * 256;
  kmax = std::max<int64_t>(kmax, 256);
  int64_t splits = std::max<int64_t>(cdiv(K, kmax), cdiv(lds_target, p.n_tiles));
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, cdiv(K, 256)));
  const int64_t kc = cdiv(cdiv(K, splits), 256) * 256;
  p.k_chunk = (int32_t)kc;
  p.splits = (int32_t)cdiv(K, kc);
  return p;
}

// Many rows (bf16): gemm_tile_kernel, 256 x bn tiles, one workgroup per CU.
// Splitting K fills more CUs but writes (and makes the consumer read) one fp32
// partial product per split; narrower tiles fill more CUs without splits but
// re-read the activation rows once per column tile and reuse each fragment
// less.  The (bn, splits) pair minimises a three-term estimate: MFMA time
// (workgroups in rounds of 256, each at a per-CU rate of 60% of the bf16 peak
// for 256-wide tiles, 55% for 128, 45% for 64), the partial traffic (8 bytes
// per output and split at 5 TB/s) and the activation re-reads (2 bytes per
// row, K-value and column tile at 20 TB/s from L2).  Chunks are whole 64-wide
// K-steps.
SkinnyPlan plan_tile(int64_t M, int64_t N, int64_t K) {
  SkinnyPlan p{};
  p.tile = true;
  p.m_tiles = (int32_t)cdiv(M, 256);
  const int64_t max_splits = std::max<int64_t>(1, std::min<int64_t>(K / 64, 32));
  const double peak_cu = 2.5e15 / 256, bw = 5e12, l2 = 20e12;
  int best_bn = 256;
  int64_t best_sp = 1;
  double best_t = 0;
  bool first = true;
  for (int bn : {256, 128, 64}) {
    const double eff = bn == 256 ? 0.6 : bn == 128 ? 0.55 : 0.45;
    const int64_t n_tiles = cdiv(N, bn);
    const int64_t tiles = (int64_t)p.m_tiles * n_tiles;
    const double tile_flops = 2.0 * 256 * bn * (double)K;
    const double reread = (double)n_tiles * p.m_tiles * 256 * K * 2 / l2;
    for (int64_t sp = 1; sp <= max_splits; ++sp) {
      const double rounds = (double)cdiv(tiles * sp, 256);
      const double t = rounds * tile_flops / sp / (peak_cu * eff) + (double)sp * M * N * 8 / bw + reread;
      if (first || t < best_t) { best_bn = bn; best_sp = sp; best_t = t; first = false; }
    }
  }
  p.tile_bn = best_bn;
  p.n_tiles = (int32_t)cdiv(N, best_bn);
  const int64_t kc = cdiv(cdiv(K, best_sp), 64) * 64;
  p.k_chunk = (int32_t)kc;
  p.splits = (int32_t)cdiv(K, kc);
  return p;
}

// Whether a bf16 product of M rows takes gemm_tile_kernel: more rows than one
// weight-streaming problem holds (which would stream the weights once per 64
// rows), K a multiple of the 64-wide step and N of 4 (row alignment follows
// from the 16-byte alignment every device pointer of the interface must have).
// Depends on shapes only, so that a workspace sized from the plan fits the
// plan the call makes.
bool tile_eligible(int64_t M, int64_t N, int64_t K, size_t eb) {
  const int64_t lo = rows_per_problem(K, eb) + 1;
  return eb == 2 && M >= lo && K % 64 == 0 && N % 4 == 0;
}

size_t lds_bytes(const GemmProb& p, size_t eb) { return (size_t)p.mt * 16 * (size_t)(p.k_chunk + 8) * eb; }


// A product of the (virtual) row concatenation [x0 (m0 rows); x1 (m1 rows)] with
// W^T, written as fp32 split-K partials [splits][M][N].  Rows are processed in
// problems of at most 64.
struct GemmJob {
  const void* x0;
  const void* x1;
  int64_t m0, m1;
  const void* w;
  int64_t N, K;
  SkinnyPlan plan;
  float* part;
  // full-K plans only: write the result in the storage type to out_final (plus
  // add, when set) instead of fp32 to part
  void* out_final = nullptr;
  const void* add = nullptr;
};

GemmJob make_job(const void* x0, int64_t m0, const void* x1, int64_t m1, const void* w, int64_t N,
                 int64_t K, size_t eb) {
  GemmJob j;
  j.x0 = x0; j.m0 = m0; j.x1 = x1; j.m1 = m1; j.w = w; j.N = N; j.K = K;
  if (tile_eligible(m0 + m1, N, K, eb))
    j.plan = plan_tile(m0 + m1, N, K);
  else
    j.plan = plan_skinny(std::min<int64_t>(m0 + m1, rows_per_problem(K, eb)), N, K, eb);
  j.part = nullptr;
  return j;
}

size_t job_part_bytes(const GemmJob& j) {
  return (size_t)j.plan.splits * (size_t)(j.m0 + j.m1) * (size_t)j.N * sizeof(float);
}

void job_problems(const GemmJob& j, size_t eb, std::vector<GemmProb>* out) {
  const int64_t M = j.m0 + j.m1;
  const int64_t step = rows_per_problem(j.K, eb);
  for (int64_t a = 0; a < M; a += step) {
    const int64_t e = std::min<int64_t>(a + step, M);
    GemmProb p{};
    const int64_t a0 = std::min(a, j.m0), e0 = std::min(e, j.m0);
    p.m0 = (int32_t)(e0 - a0);
    p.x0 = static_cast<const char*>(j.x0) + (size_t)a0 * j.K * eb;
    const int64_t a1 = std::max(a, j.m0) - j.m0, e1 = std::max(e, j.m0) - j.m0;
    p.m1 = (int32_t)(e1 - a1);
    p.x1 = j.x1 ? static_cast<const char*>(j.x1) + (size_t)a1 * j.K * eb : nullptr;
    p.w = j.w;
    p.part = j.part;
    p.row_off = (int32_t)a;
    p.m_out = (int32_t)M;
    p.N = (int32_t)j.N;
    p.K = (int32_t)j.K;
    p.k_chunk = j.plan.k_chunk;
    p.splits = j.plan.splits;
    p.mt = (int32_t)cdiv(e - a, 16);
    p.n_tiles = j.plan.n_tiles;
    p.blocks = p.n_tiles * p.splits;
    out->push_back(p);
  }
}

hipError_t run_gemms(int32_t dt, const std::vector<GemmJob>& jobs, hipStream_t s) {
  const size_t eb = elem_bytes(dt);
  std::vector<GemmProb> probs, slab_probs;
  for (const auto& j : jobs) {
    if (j.m0 + j.m1 == 0) continue;
    if (j.plan.tile) {
      TileProb t{};
      t.x0 = static_cast<const bf16*>(j.x0);
      t.x1 = static_cast<const bf16*>(j.x1);
      t.m0 = (int32_t)j.m0;
      t.m1 = (int32_t)j.m1;
      t.w = static_cast<const bf16*>(j.w);
      t.part = j.part;
      t.N = (int32_t)j.N;
      t.K = (int32_t)j.K;
      t.k_chunk = j.plan.k_chunk;
      t.splits = j.plan.splits;
      t.m_tiles = j.plan.m_tiles;
      t.n_tiles = j.plan.n_tiles;
      hipError_t e = launch_gemm_tile(t, j.plan.tile_bn, s);
      if (e != hipSuccess) return e;
      continue;
    }
    if (j.plan.resident) {
      FullkArgs f{};
      f.x0 = static_cast<const bf16*>(j.x0);
      f.x1 = static_cast<const bf16*>(j.x1);
      f.m0 = (int32_t)j.m0;
      f.m1 = (int32_t)j.m1;
      f.w = static_cast<const bf16*>(j.w);
      f.N = (int32_t)j.N;
      f.K = (int32_t)j.K;
      f.part = j.part;
      hipError_t e = launch_gemm_resident(f, s);
      if (e != hipSuccess) return e;
      continue;
    }
    if (j.plan.fullk) {
      FullkArgs f{};
      f.x0 = static_cast<const bf16*>(j.x0);
      f.x1 = static_cast<const bf16*>(j.x1);
      f.m0 = (int32_t)j.m0;
      f.m1 = (int32_t)j.m1;
      f.w = static_cast<const bf16*>(j.w);
      f.N = (int32_t)j.N;
      f.K = (int32_t)j.K;
      if (j.out_final != nullptr) {
        f.out = j.out_final;
        f.add = j.add;
      } else {
        f.part = j.part;
      }
      hipError_t e = launch_gemm_fullk(f, s);
      if (e != hipSuccess) return e;
      continue;
    }
    if (j.plan.stream) {
      TileProb t{};
      t.x0 = static_cast<const bf16*>(j.x0);
      t.x1 = static_cast<const bf16*>(j.x1);
      t.m0 = (int32_t)j.m0;
      t.m1 = (int32_t)j.m1;
      t.w = static_cast<const bf16*>(j.w);
      t.part = j.part;
      t.N = (int32_t)j.N;
      t.K = (int32_t)j.K;
      t.k_chunk = j.plan.k_chunk;
      t.splits = j.plan.splits;
      t.n_tiles = j.plan.n_tiles;
      hipError_t e = launch_gemm_stream(t, j.plan.mt, s);
      if (e != hipSuccess) return e;
      continue;
    }
    if (j.plan.wide) {
      std::vector<GemmProb> w;
      job_problems(j, eb, &w);
      for (const auto& p : w) {
        hipError_t e = launch_gemm_wide(p, s);
        if (e != hipSuccess) return e;
      }
    } else if (j.plan.slab) {
      job_problems(j, eb, &slab_probs);
    } else {
      job_problems(j, eb, &probs);
    }
  }
  // gemm_slab_kernel problems, two per launch when their row tiles agree
  for (size_t i = 0; i < slab_probs.size();) {
    GemmArgs a{};
    a.p[0] = slab_probs[i];
    a.nprob = 1;
    size_t lds = lds_bytes(slab_probs[i], eb);
    if (i + 1 < slab_probs.size() && slab_probs[i + 1].mt == slab_probs[i].mt) {
      a.p[1] = slab_probs[i + 1];
      a.nprob = 2;
      lds = std::max(lds, lds_bytes(slab_probs[i + 1], eb));
    }
    i += a.nprob;
    hipError_t e = launch_gemm_slab(a, lds, s);
    if (e != hipSuccess) return e;
  }
  // gemm_lds_kernel problems, two per launch
  for (size_t i = 0; i < probs.size(); i += 2) {
    GemmArgs a{};
    a.p[0] = probs[i];
    a.nprob = 1;
    int max_mt = probs[i].mt;
    size_t lds = lds_bytes(probs[i], eb);
    if (i + 1 < probs.size()) {
      a.p[1] = probs[i + 1];
      a.nprob = 2;
      max_mt = std::max(max_mt, probs[i + 1].mt);
      lds = std::max(lds, lds_bytes(probs[i + 1], eb));
    }
    hipError_t e = launch_gemm_lds(dt, a, max_mt, lds, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- cache helpers

// len_s = new_len[s] (0 <= new_len[s] <= len_s, checked by the caller);
// pages at or past ceil(new_len / page_size) return to the free list.
void crop_host(dflash_cache* c, const int32_t* new_len) {
  for (int s = 0; s < c->desc.n_seqs; ++s) {
    c->len[s] = new_len[s];
    if (c->desc.page_size > 0) {
      const size_t keep = (size_t)cdiv(new_len[s], c->desc.page_size);
      for (size_t j = keep; j < c->pages[s].size(); ++j) c->free_pages.insert(c->pages[s][j]);
      c->pages[s].resize(std::min(keep, c->pages[s].size()));
    }
  }
}

CacheView view_of(const dflash_cache* c) {
  CacheView v{};
  v.k_pool = c->desc.k_pool;
  v.v_pool = c->desc.v_pool;
  v.block_table = c->desc.page_size > 0 ? c->desc.block_table : nullptr;
  v.page_rows = c->desc.page_size > 0 ? c->desc.page_size : (int32_t)c->desc.capacity;
  v.max_pages = c->desc.page_size > 0 ? c->desc.max_pages_per_seq : 1;
  v.n_kv = c->desc.n_kv;
  v.d_h = c->desc.d_h;
  return v;
}

// New pages an append of n[s] rows per sequence needs; checks every limit.
struct AppendPlan {
  std::vector<std::vector<int32_t>> new_pages;   // per sequence, in logical order
};

int plan_append(const dflash_cache* c, const std::vector<int64_t>& n, AppendPlan* plan) {
  const auto& d = c->desc;
  plan->new_pages.assign(d.n_seqs, {});
  if (d.page_size == 0) {
    // a ring takes any length, at most `capacity` new rows per call (more
    // would land twice in one slot)
    for (int s = 0; s < d.n_seqs; ++s)
      if (d.ring ? n[s] > d.capacity : c->len[s] + n[s] > d.capacity) return DFLASH_ERR_CAPACITY;
    return DFLASH_OK;
  }
  int64_t need = 0;
  for (int s = 0; s < d.n_seqs; ++s) {
    const int64_t want = cdiv(c->len[s] + n[s], d.page_size);
    if (want > d.max_pages_per_seq) return DFLASH_ERR_CAPACITY;
    need += std::max<int64_t>(0, want - (int64_t)c->pages[s].size());
  }
  if (need > (int64_t)c->free_pages.size()) return DFLASH_ERR_CAPACITY;
  auto it = c->free_pages.begin();
  for (int s = 0; s < d.n_seqs; ++s) {
    const int64_t want = cdiv(c->len[s] + n[s], d.page_size);
    for (int64_t j = (int64_t)c->pages[s].size(); j < want; ++j) plan->new_pages[s].push_back(*it++);
  }
  return DFLASH_OK;
}

hipError_t enqueue_page_table_now(const dflash_cache* c, const AppendPlan& plan, hipStream_t st);

hipError_t enqueue_page_table(const dflash_cache* c, const AppendPlan& plan, hipStream_t st) {
  const auto& d = c->desc;
  if (d.page_size == 0) return hipSuccess;
  size_t total = 0;
  for (const auto& v : plan.new_pages) total += v.size();
  if (total == 0) return hipSuccess;
  return staged(DFLASH_STAGE_PAGE_TABLE, st, true, [&] { return enqueue_page_table_now(c, plan, st); });
}

hipError_t enqueue_page_table_now(const dflash_cache* c, const AppendPlan& plan, hipStream_t st) {
  const auto& d = c->desc;
  BtUpdateArgs a{};
  a.table = d.block_table;
  for (int s = 0; s < d.n_seqs; ++s) {
    const int32_t first = (int32_t)c->pages[s].size();
    for (size_t j = 0; j < plan.new_pages[s].size(); ++j) {
      a.index[a.count] = s * d.max_pages_per_seq + first + (int32_t)j;
      a.value[a.count] = plan.new_pages[s][j];
      if (++a.count == kBtBatch) {
        hipError_t e = launch_bt_update(a, st);
        if (e != hipSuccess) return e;
        a.count = 0;
      }
    }
  }
  return launch_bt_update(a, st);
}

void commit_append(dflash_cache* c, const std::vector<int64_t>& n, const AppendPlan& plan) {
  for (int s = 0; s < c->desc.n_seqs; ++s) {
    c->len[s] += (int32_t)n[s];
    c->written_hi[s] = std::max<int64_t>(c->written_hi[s], c->len[s]);
    for (int32_t pg : plan.new_pages[s]) {
      c->free_pages.erase(pg);
      c->pages[s].push_back(pg);
    }
  }
}

int check_cu(const int32_t* cu, int n_seqs, std::vector<int64_t>* n) {
  if (!cu || cu[0] != 0) return DFLASH_ERR_ARG;
  n->resize(n_seqs);
  for (int s = 0; s < n_seqs; ++s) {
    if (cu[s + 1] < cu[s]) return DFLASH_ERR_ARG;
    (*n)[s] = cu[s + 1] - cu[s];
  }
  return DFLASH_OK;
}

// ---------------------------------------------------------------- layer planning

int check_layer(const dflash_layer_desc* L) {
  if (!L) return DFLASH_ERR_ARG;
  if (!dtype_ok(L->dtype)) return DFLASH_ERR_DTYPE;
  if (L->d <= 0 || L->n_h <= 0 || L->n_kv <= 0 || L->n_h % L->n_kv != 0) return DFLASH_ERR_SHAPE;
  if (L->d_h != 64 && L->d_h != 128) return DFLASH_ERR_SHAPE;
  if (L->d % 8 != 0 || L->window < 0 || !(L->eps >= 0.f) || !(L->rope_theta > 0.0)) return DFLASH_ERR_SHAPE;
  if (L->residual != 0 && L->residual != 1) return DFLASH_ERR_ARG;
  if (!L->w_qkv || !L->w_o || !L->gamma_q || !L->gamma_k) return DFLASH_ERR_ARG;
  if (!aligned16(L->w_qkv) || !aligned16(L->w_o)) return DFLASH_ERR_ARG;
  return DFLASH_OK;
}

struct KvPlan {
  int64_t R, B, T, RB, qd, kvd, group, qrows;
  // fused_qkv: one product of [C; H] with all of W_qkv (Q columns of the C
  // rows are computed and ignored) when every row fits one weight-streaming
  // problem - the weights are then streamed once, in one launch; otherwise Q
  // of H and K/V of [C; H] as two products (gq, gkv).
  // block_rows_apart: instead, Q, K and V of H in one weight-streaming
  // product (gq) and K/V of C alone (gkv), when the block rows would add a
  // 256-row tile to a tile-GEMM K/V product (1024 fresh context rows + 16
  // block rows: 5 row tiles, the fifth holding 16 rows).
  bool fused_qkv;
  bool block_rows_apart;
  GemmJob gq, gkv, go;
  size_t off_q, off_pq, off_pkv, off_po, off_pml, off_attn, off_pout, off_sync, total;
  int64_t max_items;
};

// items_exact >= 0 sizes the attention partials for exactly that many work
// items (a call whose split is known); otherwise for the most any call with
// these sizes may plan.
KvPlan plan_kv(const dflash_layer_desc* L, const dflash_cache* c, int64_t T, int32_t B, int64_t items_exact = -1) {
  KvPlan p{};
  const size_t eb = elem_bytes(L->dtype);
  p.R = c->desc.n_seqs; p.B = B; p.T = T; p.RB = p.R * B;
  p.qd = (int64_t)L->n_h * L->d_h;
  p.kvd = (int64_t)L->n_kv * L->d_h;
  p.group = L->n_h / L->n_kv;
  p.qrows = cdiv(p.group * B, 16) * 16;
  // one [C; H] product with all of w_qkv up to 64 rows (the Q columns of the
  // context rows cost nothing next to streaming the weights once); beyond,
  // Q of the block rows and K/V of all rows separately (the fused product's
  // split-K partials would be 1.5x the two separate ones')
  p.fused_qkv = T + p.RB <= std::min<int64_t>(kSkinnyMaxM, rows_per_problem(L->d, eb));
  if (p.fused_qkv) {
    p.gkv = make_job(nullptr, T, nullptr, p.RB, L->w_qkv, p.qd + 2 * p.kvd, L->d, eb);
    p.gq = p.gkv;
    p.gq.plan.splits = 0;   // no separate partials
  } else {
    constexpr int64_t kTileRows = 256;
    p.block_rows_apart = p.RB <= kSkinnyMaxM && tile_eligible(T, 2 * p.kvd, L->d, eb) &&
                         cdiv(T + p.RB, kTileRows) > cdiv(T, kTileRows);
    if (p.block_rows_apart) {
      p.gq = make_job(nullptr, 0, nullptr, p.RB, L->w_qkv, p.qd + 2 * p.kvd, L->d, eb);
      p.gkv = make_job(nullptr, T, nullptr, 0, nullptr, 2 * p.kvd, L->d, eb);
    } else {
      p.gq = make_job(nullptr, 0, nullptr, p.RB, L->w_qkv, p.qd, L->d, eb);
      p.gkv = make_job(nullptr, T, nullptr, p.RB, nullptr, 2 * p.kvd, L->d, eb);
    }
  }
  p.go = make_job(nullptr, p.RB, nullptr, 0, L->w_o, L->d, p.qd, eb);
  // work items of one attention launch: at most the target count plus one
  // partial chunk per (sequence, head); on a paged cache the chunk may be capped
  // at (kAttnMaxChunkPages - 2) pages, and the keys of all sequences fit in the
  // pool, which bounds the extra items
  p.max_items = kAttnMaxTarget + 2 * p.R * L->n_kv;
  if (c->desc.page_size > 0) p.max_items += cdiv(c->desc.capacity * L->n_kv, kAttnMaxChunkPages - 2);
  if (items_exact >= 0) p.max_items = items_exact;
  size_t o = 0;
  p.off_q = o;   o = align_up(o + (size_t)p.R * L->n_kv * p.qrows * L->d_h * eb);
  p.off_pq = o;  o = align_up(o + (p.fused_qkv ? 0 : job_part_bytes(p.gq)));
  p.off_pkv = o; o = align_up(o + job_part_bytes(p.gkv));
  p.off_po = o;  o = align_up(o + (size_t)p.max_items * p.qrows * L->d_h * sizeof(float));
  p.off_pml = o; o = align_up(o + (size_t)p.max_items * 2 * p.qrows * sizeof(float));
  p.off_attn = o; o = align_up(o + (size_t)p.RB * p.qd * eb);
  p.off_pout = o; o = align_up(o + job_part_bytes(p.go));
  p.off_sync = o; o = align_up(o + (size_t)kAttnSyncStride * sizeof(uint32_t) * L->n_kv);
  p.total = o;
  return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP; }

// max of f(t) over t = 0 .. T: plans are evaluated for every row count up to
// 65536 (host arithmetic only) and for T itself beyond that, where every
// product takes the tile GEMM and its partials grow with the rows.
template <class F>
size_t max_over_rows(int64_t T, F&& f) {
  size_t m = f(T);
  for (int64_t t = 0; t < std::min<int64_t>(T, 65536); ++t) m = std::max(m, f(t));
  return m;
}

}  // namespace

// ======================================================================== ABI

extern "C" {

const char* dflash_strerror(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_ARG: return "invalid argument (null/misaligned pointer, bad handle or offsets)";
    case DFLASH_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DFLASH_ERR_DTYPE: return "unsupported dtype or dtype mismatch";
    case DFLASH_ERR_RANGE: return "crop length outside [0, current length]";
    case DFLASH_ERR_CAPACITY: return "cache capacity, page table or page pool exhausted";
    case DFLASH_ERR_HIP: return "HIP runtime error";
    case DFLASH_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int dflash_cache_init(dflash_cache** out, const dflash_cache_desc* desc) {
  if (!out || !desc) return DFLASH_ERR_ARG;
  const auto& d = *desc;
  if (!cache_dtype_ok(d.dtype)) return DFLASH_ERR_DTYPE;
  if (d.dtype == DFLASH_FP8_E4M3 && (!scale_ok(d.k_scale) || !scale_ok(d.v_scale))) return DFLASH_ERR_ARG;
  if (d.n_seqs < 1 || d.n_seqs > DFLASH_MAX_SEQS || d.n_kv < 1 || d.d_h < 8 || d.d_h % 8 != 0)
    return DFLASH_ERR_SHAPE;
  if (d.page_size < 0 || d.page_size % DFLASH_KEY_ALIGN != 0 || d.capacity <= 0) return DFLASH_ERR_SHAPE;
  if (d.page_size == 0 && (d.capacity % DFLASH_KEY_ALIGN != 0 || d.capacity > (int64_t)1 << 30))
    return DFLASH_ERR_SHAPE;
  if (d.page_size > 0 && (d.max_pages_per_seq < 1 || d.capacity > (int64_t)1 << 30)) return DFLASH_ERR_SHAPE;
  if (d.ring != 0 && (d.ring != 1 || d.page_size != 0)) return DFLASH_ERR_SHAPE;
  if (!d.k_pool || !d.v_pool || !aligned16(d.k_pool) || !aligned16(d.v_pool)) return DFLASH_ERR_ARG;
  if (d.page_size > 0 && (!d.block_table || (reinterpret_cast<uintptr_t>(d.block_table) & 3)))
    return DFLASH_ERR_ARG;
  auto* c = new dflash_cache;
  c->desc = d;
  c->len.assign(d.n_seqs, 0);
  c->written_hi.assign(d.n_seqs, 0);
  c->pages.assign(d.n_seqs, {});
  if (d.page_size > 0)
    for (int64_t i = 0; i < d.capacity; ++i) c->free_pages.insert(c->free_pages.end(), (int32_t)i);
  *out = c;
  return DFLASH_OK;
}

int dflash_cache_destroy(dflash_cache* c) {
  if (!c) return DFLASH_ERR_ARG;
  delete c;
  return DFLASH_OK;
}

int dflash_cache_lengths(const dflash_cache* c, int32_t* host_len) {
  if (!c || !host_len) return DFLASH_ERR_ARG;
  std::copy(c->len.begin(), c->len.end(), host_len);
  return DFLASH_OK;
}

int dflash_cache_block_table(const dflash_cache* c, int32_t* t) {
  if (!c || !t) return DFLASH_ERR_ARG;
  const int mp = c->desc.page_size > 0 ? c->desc.max_pages_per_seq : 1;
  for (int s = 0; s < c->desc.n_seqs; ++s)
    for (int j = 0; j < mp; ++j) {
      int32_t v = -1;
      if (c->desc.page_size == 0) v = j == 0 ? s : -1;
      else if (j < (int)c->pages[s].size()) v = c->pages[s][j];
      t[s * mp + j] = v;
    }
  return DFLASH_OK;
}

int64_t dflash_cache_free_pages(const dflash_cache* c) {
  if (!c) return DFLASH_ERR_ARG;
  return (int64_t)c->free_pages.size();
}

int dflash_cache_append(dflash_cache* c, const int32_t* cu_rows, const void* k_rows, const void* v_rows,
                        void* stream) {
  if (!c || c->dev) return DFLASH_ERR_ARG;
  std::vector<int64_t> n;
  int st = check_cu(cu_rows, c->desc.n_seqs, &n);
  if (st) return st;
  const int64_t n_rows = cu_rows[c->desc.n_seqs];
  if (n_rows > 0 && (!k_rows || !v_rows || !aligned16(k_rows) || !aligned16(v_rows))) return DFLASH_ERR_ARG;
  AppendPlan plan;
  st = plan_append(c, n, &plan);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = enqueue_page_table(c, plan, s);
  if (e == hipSuccess && n_rows > 0) {
    AppendArgs a{};
    a.k_rows = k_rows;
    a.v_rows = v_rows;
    a.cache = view_of(c);
    // the kernel sees the page table including this call's new pages
    a.n_seqs = c->desc.n_seqs;
    for (int i = 0; i < c->desc.n_seqs; ++i) a.L[i] = c->len[i];
    for (int i = 0; i <= c->desc.n_seqs; ++i) a.cu[i] = cu_rows[i];
    e = staged(DFLASH_STAGE_CACHE_APPEND, s, true,
               [&] { return launch_cache_append(c->desc.dtype, a, n_rows, s); });
  }
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  commit_append(c, n, plan);
  return DFLASH_OK;
}

int dflash_cache_crop(dflash_cache* c, const int32_t* new_len, void* /*stream*/) {
  if (!c || !new_len || c->dev) return DFLASH_ERR_ARG;
  for (int s = 0; s < c->desc.n_seqs; ++s)
    if (new_len[s] < 0 || new_len[s] > c->len[s]) return DFLASH_ERR_RANGE;
  crop_host(c, new_len);
  return DFLASH_OK;
}

size_t dflash_ctx_project_ws_bytes(int64_t T, int64_t kd, int64_t d, int32_t dtype) {
  if (T <= 0 || kd <= 0 || d <= 0 || !dtype_ok(dtype)) return 0;
  // enough for every row count up to T: the GEMM plan (and its split count)
  // changes with the rows, so fewer rows may need more partials
  return max_over_rows(T, [&](int64_t t) {
    GemmJob j = make_job(nullptr, t, nullptr, 0, nullptr, d, kd, elem_bytes(dtype));
    return align_up(job_part_bytes(j));
  });
}

int dflash_ctx_project(const void* x_raw, int64_t T, int64_t kd, const void* w_fc, const void* gamma_h,
                       int64_t d, float eps, int32_t dtype, void* c_out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (!dtype_ok(dtype)) return DFLASH_ERR_DTYPE;
  if (T < 0 || kd <= 0 || d <= 0 || kd % 8 != 0 || d % 8 != 0 || kd > INT32_MAX / 2 || d > 16384 ||
      T > INT32_MAX / 2 || !(eps >= 0.f))
    return DFLASH_ERR_SHAPE;
  if (T == 0) return DFLASH_OK;
  if (!x_raw || !w_fc || !gamma_h || !c_out || !ws) return DFLASH_ERR_ARG;
  if (!aligned16(x_raw) || !aligned16(w_fc) || !aligned16(c_out) || !aligned16(ws)) return DFLASH_ERR_ARG;
  if (ws_bytes < dflash_ctx_project_ws_bytes(T, kd, d, dtype)) return DFLASH_ERR_WORKSPACE;
  const size_t eb = elem_bytes(dtype);
  GemmJob j = make_job(x_raw, T, nullptr, 0, w_fc, d, kd, eb);
  j.part = static_cast<float*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = staged(DFLASH_STAGE_CTX_GEMM, s, true, [&] { return run_gemms(dtype, {j}, s); });
  if (e == hipSuccess)
    e = staged(DFLASH_STAGE_CTX_NORM, s, true, [&] {
      return launch_reduce_rmsnorm(dtype, j.part, j.plan.splits, T, d, gamma_h, eps, c_out, s);
    });
  return hip_status(e);
}

size_t dflash_kv_inject_attn_ws_bytes(const dflash_layer_desc* L, const dflash_cache* c, int64_t T, int32_t B) {
  if (check_layer(L) != DFLASH_OK || !c || T < 0 || B < 1) return 0;
  // enough for every context row count up to T (see dflash_ctx_project_ws_bytes)
  return max_over_rows(T, [&](int64_t t) { return plan_kv(L, c, t, B).total; });
}

}  // extern "C"

namespace {

// Compute units of the current device (0 if it cannot be queried), read once
// per device.
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = n;
  }
  return cus[dev];
}

// One layer call.  exact_ws: the workspace must hold this call's own needs
// (the attention partials of its planned split), not the figure that holds
// for every call with these sizes.
// dev_rows (device [n_seqs]): a device-driven round of the cache's device
// mode; cu_ctx then holds the fixed stride n_max (cu_ctx[r] = r * n_max) and
// every bound below is planned for n_max new rows per sequence.
int kv_inject_impl(const dflash_layer_desc* L, dflash_cache* c, const void* C, const int32_t* cu_ctx,
                   const void* H, int32_t B, void* out, void* ws, size_t ws_bytes, void* stream, bool exact_ws,
                   const int32_t* dev_rows = nullptr) {
  int st = check_layer(L);
  if (st) return st;
  if (!c) return DFLASH_ERR_ARG;
  // a cache in device mode takes device-driven rounds only (its host
  // lengths are bounds), and device-driven rounds need device mode
  if (c->dev != (dev_rows != nullptr)) return DFLASH_ERR_ARG;
  const auto& cd = c->desc;
  const bool fp8 = cd.dtype == DFLASH_FP8_E4M3;
  if (cd.dtype != L->dtype && !(fp8 && L->dtype == DFLASH_BF16)) return DFLASH_ERR_DTYPE;
  if (cd.n_kv != L->n_kv || cd.d_h != L->d_h) return DFLASH_ERR_SHAPE;
  if (B < 1 || (int64_t)(L->n_h / L->n_kv) * B > DFLASH_MAX_GROUP_ROWS) return DFLASH_ERR_SHAPE;
  std::vector<int64_t> n;
  st = check_cu(cu_ctx, cd.n_seqs, &n);
  if (st) return st;
  const int64_t T = cu_ctx[cd.n_seqs];
  if (T > 0 && (!C || !aligned16(C))) return DFLASH_ERR_ARG;
  if (!H || !out || !ws || !aligned16(H) || !aligned16(out) || !aligned16(ws)) return DFLASH_ERR_ARG;
  KvPlan p = plan_kv(L, c, T, B);
  if (!exact_ws && ws_bytes < p.total) return DFLASH_ERR_WORKSPACE;
  std::vector<int64_t> rows(cd.n_seqs);
  for (int s = 0; s < cd.n_seqs; ++s) rows[s] = n[s] + B;
  if (cd.ring && dev_rows != nullptr) return DFLASH_ERR_SHAPE;
  if (cd.ring) {
    // a ring holds the last `capacity` positions: the window and the new rows
    // must fit, and every key the window reaches must still be held
    if (L->window <= 0) return DFLASH_ERR_SHAPE;
    if (cd.capacity < (int64_t)L->window + B - 1) return DFLASH_ERR_CAPACITY;
    for (int s = 0; s < cd.n_seqs; ++s) {
      const int64_t lo = std::max<int64_t>(0, c->len[s] + n[s] - L->window + 1);
      if (lo < c->written_hi[s] - cd.capacity) return DFLASH_ERR_RANGE;
    }
  }
  AppendPlan ap;
  st = plan_append(c, rows, &ap);
  if (st) return st;

  const int32_t dt = L->dtype;
  const int R = cd.n_seqs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t eb = elem_bytes(dt);

  // the attention split, planned before anything is enqueued (every key of
  // every sequence after this call's append)
  AttnArgs aa{};
  aa.cache = view_of(c);
  aa.R = R; aa.B = B; aa.n_kv = L->n_kv; aa.group = (int32_t)p.group; aa.qrows = (int32_t)p.qrows;
  aa.d_h = L->d_h; aa.window = L->window;
  // an fp8 cache's key scale multiplies every score: it joins the softmax
  // scale; its value scale multiplies every output (applied to the partials)
  aa.scale_log2 = (float)(1.0 / std::sqrt((double)L->d_h) * 1.4426950408889634 * (fp8 ? cd.k_scale : 1.0));
  aa.v_scale = fp8 ? cd.v_scale : 1.f;
  if (dev_rows != nullptr) {
    aa.d_len = c->d_len;
    aa.d_rows = dev_rows;
    aa.n_max = cu_ctx[1];
  }
  int64_t items = 0;
  {
    std::vector<int64_t> keys(R);
    for (int r = 0; r < R; ++r) {
      const int64_t hi = c->len[r] + n[r] + B;
      const int64_t lo = L->window > 0 ? std::max<int64_t>(0, c->len[r] + n[r] - L->window + 1) : 0;
      aa.key_hi[r] = (int32_t)hi;
      aa.key_lo[r] = (int32_t)lo;
      aa.qpos0[r] = (int32_t)(c->len[r] + n[r]);
      keys[r] = hi - (lo & ~int64_t(63));
      // device-driven rounds: the true window start lies anywhere below the
      // bound, and a window (from its block-aligned start) spans at most
      // window + B + 62 keys
      if (dev_rows != nullptr && L->window > 0) keys[r] = std::min<int64_t>(hi, (int64_t)L->window + B + 62);
    }
    // an item's keys may span at most kAttnMaxChunkPages pages (its page list
    // is staged in LDS); two pages go to a chunk that does not start on a page.
    // A ring's positions wrap every `capacity` rows: each wrap an item spans
    // takes one more entry of its page list.
    int64_t cap = (int64_t)1 << 30;
    if (cd.page_size > 0) cap = std::min<int64_t>(cap, (int64_t)(kAttnMaxChunkPages - 2) * cd.page_size);
    if (cd.ring) cap = std::min<int64_t>(cap, (int64_t)(kAttnMaxChunkPages - 2) * cd.capacity);
    const AttnSplit sp = plan_attn_split(keys, L->n_kv, cap, fp8);
    aa.nst = sp.nst;
    // each item starts its blocks at (item * 37) mod its block count: with
    // every item starting at block 0, the items running at once stream
    // regularly spaced addresses in step (a 4 x 33K batch: 125 -> 110 us)
    aa.rot = 37;
    aa.chunk_keys = (int32_t)sp.chunk;
    for (int r = 0; r < R; ++r) {
      aa.item_base[r] = (int32_t)items;
      aa.chunks[r] = (int32_t)std::max<int64_t>(1, cdiv(keys[r], sp.chunk));
      items += (int64_t)aa.chunks[r] * L->n_kv;
    }
    aa.item_base[R] = (int32_t)items;
    aa.seq0[0] = aa.key_lo[0];
    aa.seq0[1] = aa.key_hi[0];
    aa.seq0[2] = aa.qpos0[0];
    aa.seq0[3] = aa.chunks[0];
    // bounded by construction for the planner's splits; a forced split may not fit
    if (items > p.max_items) return DFLASH_ERR_SHAPE;
  }
  // The split merges in the attention launch itself (no combine launch) for
  // one sequence of bf16 rows over a bf16 or fp8 cache with 49..64 query rows
  // per K/V head at d_h 128, on the one-workgroup-per-CU plans: the items of a
  // head wait for each other, so every item must be resident at once (at
  // most one per compute unit), and a head's items must share an XCD (n_kv
  // a multiple of the 8 XCDs; item x takes head x % n_kv), at most
  // kAttnMergeMaxItems of them (one arrival flag each).  Device-driven
  // rounds keep the combine launch, which also advances the device lengths.
  const bool merge_in_attn = dt == DFLASH_BF16 && L->d_h == 128 && cdiv(p.qrows, 16) == 4 &&
                             aa.nst >= 3 && R == 1 && L->n_kv % 8 == 0 && L->n_kv <= 64 && dev_rows == nullptr && items > 0 &&
                             items <= device_cus() && aa.chunks[0] <= kAttnMergeMaxItems;
  if (exact_ws) {
    p = plan_kv(L, c, T, B, items);
    if (ws_bytes < p.total) return DFLASH_ERR_WORKSPACE;
  }
  char* w = static_cast<char*>(ws);
  void* q_ws = w + p.off_q;
  float* part_q = reinterpret_cast<float*>(w + p.off_pq);
  float* part_kv = reinterpret_cast<float*>(w + p.off_pkv);
  float* part_o = reinterpret_cast<float*>(w + p.off_po);
  float* part_ml = reinterpret_cast<float*>(w + p.off_pml);
  void* attn = w + p.off_attn;
  float* part_out = reinterpret_cast<float*>(w + p.off_pout);
  aa.q_ws = q_ws; aa.part_o = part_o; aa.part_ml = part_ml;
  uint32_t* attn_sync = reinterpret_cast<uint32_t*>(w + p.off_sync);
  if (merge_in_attn) {
    aa.sync = attn_sync;
    aa.attn = attn;
    aa.merge_spread = g_merge_spread.load();
    aa.spin_limit = g_spin_limit.load();
  }

  // 1. page table entries for the rows this call appends
  hipError_t e = enqueue_page_table(c, ap, s);

  // 2. q/k/v projection: Q from the block rows, K/V from [C; H] with one weight
  //    (the block rows' K/V in their Q product when block_rows_apart)
  GemmJob gq = p.gq, gkv = p.gkv;
  gkv.x0 = C; gkv.x1 = H; gkv.part = part_kv;
  if (p.fused_qkv) {
    if (e == hipSuccess) e = staged(DFLASH_STAGE_QKV_GEMM, s, true, [&] { return run_gemms(dt, {gkv}, s); });
  } else {
    gq.x1 = H; gq.part = part_q;
    gkv.w = static_cast<const char*>(L->w_qkv) + (size_t)p.qd * L->d * eb;
    if (e == hipSuccess) e = staged(DFLASH_STAGE_QKV_GEMM, s, true, [&] { return run_gemms(dt, {gq, gkv}, s); });
  }

  // 3. norms, RoPE, Q to the workspace, K/V into the cache
  CacheView cv = view_of(c);
  if (e == hipSuccess) {
    QkvEpiArgs a{};
    if (p.fused_qkv) {
      // [splits][T + RB][qd + 2 kvd]: Q of the block rows at rows T.., K/V after column qd
      const int64_t w = p.qd + 2 * p.kvd, split = (T + p.RB) * w;
      a.part_q = part_kv + T * w;
      a.q_row = w; a.q_split = split;
      a.part_kv = part_kv + p.qd;
      a.kv_row = w; a.kv_split = split;
      a.sq = a.skv = gkv.plan.splits;
      a.part_kvh = a.part_kv + T * w;
      a.kvh_row = w; a.kvh_split = split; a.skvh = a.skv;
    } else if (p.block_rows_apart) {
      // [splits][RB][qd + 2 kvd] for the block rows, [splits][T][2 kvd] for C
      const int64_t w = p.qd + 2 * p.kvd;
      a.part_q = part_q;
      a.q_row = w; a.q_split = p.RB * w;
      a.part_kv = part_kv;
      a.kv_row = 2 * p.kvd; a.kv_split = T * 2 * p.kvd;
      a.sq = gq.plan.splits; a.skv = gkv.plan.splits;
      a.part_kvh = part_q + p.qd;
      a.kvh_row = w; a.kvh_split = p.RB * w; a.skvh = gq.plan.splits;
    } else {
      a.part_q = part_q;
      a.q_row = p.qd; a.q_split = p.RB * p.qd;
      a.part_kv = part_kv;
      a.kv_row = 2 * p.kvd; a.kv_split = (T + p.RB) * 2 * p.kvd;
      a.sq = gq.plan.splits; a.skv = gkv.plan.splits;
      a.part_kvh = part_kv + T * a.kv_row;
      a.kvh_row = a.kv_row; a.kvh_split = a.kv_split; a.skvh = a.skv;
    }
    a.gamma_q = L->gamma_q; a.gamma_k = L->gamma_k;
    a.q_ws = q_ws;
    a.cache = cv;
    a.R = R; a.B = B; a.T = (int32_t)T; a.n_h = L->n_h; a.n_kv = L->n_kv; a.d_h = L->d_h;
    a.qrows = (int32_t)p.qrows;
    a.eps = L->eps;
    for (int i = 0; i < L->d_h / 2; ++i) a.inv_freq[i] = std::pow(L->rope_theta, -2.0 * i / L->d_h);
    for (int r = 0; r < R; ++r) { a.seq.L[r] = c->len[r]; a.seq.n[r] = (int32_t)n[r]; }
    for (int r = 0; r <= R; ++r) a.seq.cu[r] = cu_ctx[r];
    a.cache_fp8 = fp8 ? 1 : 0;
    a.k_scale = fp8 ? cd.k_scale : 1.f;
    a.v_scale = fp8 ? cd.v_scale : 1.f;
    if (dev_rows != nullptr) {
      a.d_len = c->d_len;
      a.d_rows = dev_rows;
      a.n_max = cu_ctx[1];
    }
    if (merge_in_attn) {
      a.attn_sync = attn_sync;
      a.n_sync = L->n_kv;
    }
    e = staged(DFLASH_STAGE_QKV_EPILOGUE, s, true, [&] { return launch_qkv_epilogue(dt, a, s); });
  }

  // 4. attention over every cached key, split into chunks, and the merge
  {
    if (e == hipSuccess)
      e = staged(DFLASH_STAGE_ATTN, s, items > 0, [&] {
        return fp8 ? launch_attn_fp8(aa, (int)items, s) : launch_attn_split(dt, aa, (int)items, s);
      });
    if (e == hipSuccess && !merge_in_attn) {
      CombineArgs ca{};
      ca.part_o = part_o; ca.part_ml = part_ml; ca.attn = attn;
      ca.R = R; ca.B = B; ca.n_kv = L->n_kv; ca.group = (int32_t)p.group; ca.qrows = (int32_t)p.qrows;
      ca.d_h = L->d_h;
      if (dev_rows != nullptr) {
        ca.d_len = c->d_len;
        ca.d_rows = dev_rows;
        ca.n_max = cu_ctx[1];
      }
      for (int r = 0; r <= R; ++r) ca.item_base[r] = aa.item_base[r];
      for (int r = 0; r < R; ++r) ca.chunks[r] = aa.chunks[r];
      e = staged(DFLASH_STAGE_ATTN_COMBINE, s, true, [&] { return launch_attn_combine(dt, ca, s); });
    }
  }

  // 5. o_proj
  GemmJob go = p.go;
  go.x0 = attn; go.part = part_out;
  if (go.plan.fullk) {
    // one result per output: o_proj (plus the residual) straight into out
    go.out_final = out;
    go.add = L->residual ? H : nullptr;
  }
  if (e == hipSuccess) e = staged(DFLASH_STAGE_O_GEMM, s, true, [&] { return run_gemms(dt, {go}, s); });
  if (e == hipSuccess && !go.plan.fullk)
    e = staged(DFLASH_STAGE_O_REDUCE, s, true,
               [&] {
                 return launch_splitk_reduce(dt, part_out, go.plan.splits, p.RB, L->d, L->residual ? H : nullptr,
                                             out, s);
               });
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  commit_append(c, rows, ap);
  return DFLASH_OK;
}

// The scratch buffer of dflash_kv_inject_attn_noalloc: device memory of the
// library's own, one copy per GPU for the life of the process.  In host code
// `scratch` names a host-side stand-in; the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is ever handed to kernels.
constexpr size_t kScratchBytes = (size_t)DFLASH_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_address(int* status) {
  static std::mutex mu;
  static void* ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    *status = DFLASH_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> g(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *status = DFLASH_ERR_HIP;
      return nullptr;
    }
    ptr[dev] = p;
  }
  *status = DFLASH_OK;
  return ptr[dev];
}

}  // namespace

extern "C" {

int dflash_kv_inject_attn(const dflash_layer_desc* L, dflash_cache* c, const void* C, const int32_t* cu_ctx,
                          const void* H, int32_t B, void* out, void* ws, size_t ws_bytes, void* stream) {
  return kv_inject_impl(L, c, C, cu_ctx, H, B, out, ws, ws_bytes, stream, false);
}

size_t dflash_kv_inject_attn_dev_ws_bytes(const dflash_layer_desc* L, const dflash_cache* c, int32_t n_max,
                                          int32_t B) {
  if (!c || n_max < 0) return 0;
  return dflash_kv_inject_attn_ws_bytes(L, c, (int64_t)c->desc.n_seqs * n_max, B);
}

int dflash_kv_inject_attn_dev(const dflash_layer_desc* L, dflash_cache* c, const void* C, int32_t n_max,
                              const int32_t* d_rows, const void* H, int32_t B, void* out, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!c || !d_rows || (reinterpret_cast<uintptr_t>(d_rows) & 3)) return DFLASH_ERR_ARG;
  if (n_max < 0 || n_max > (1 << 20)) return DFLASH_ERR_SHAPE;
  std::vector<int32_t> cu(c->desc.n_seqs + 1);
  for (int r = 0; r <= c->desc.n_seqs; ++r) cu[r] = r * n_max;
  return kv_inject_impl(L, c, C, cu.data(), H, B, out, ws, ws_bytes, stream, false, d_rows);
}

int dflash_kv_inject_attn_noalloc(const dflash_layer_desc* L, dflash_cache* c, const void* C,
                                  const int32_t* cu_ctx, const void* H, int32_t B, void* out, void* stream) {
  int st = DFLASH_OK;
  void* ws = scratch_address(&st);
  if (st) return st;
  const bool was = t_untimed;
  t_untimed = true;
  st = kv_inject_impl(L, c, C, cu_ctx, H, B, out, ws, kScratchBytes, stream, true);
  t_untimed = was;
  return st;
}

// ---------------------------------------------------------------- draft head

}  // extern "C"

namespace {
struct HeadPlan {
  int64_t M;
  GemmJob j;
  int nseg;
  size_t off_x, off_part, off_val, off_idx, total;
};

HeadPlan plan_head(int64_t R, int32_t B, int64_t d, int64_t vocab, size_t eb) {
  HeadPlan p{};
  p.M = R * (B - 1);
  p.j = make_job(nullptr, p.M, nullptr, 0, nullptr, vocab, d, eb);
  p.nseg = (int)cdiv(vocab, kHeadSeg);
  size_t o = 0;
  p.off_x = o;    o = align_up(o + (size_t)p.M * d * eb);
  p.off_part = o; o = align_up(o + job_part_bytes(p.j));
  p.off_val = o;  o = align_up(o + (size_t)p.M * p.nseg * sizeof(float));
  p.off_idx = o;  o = align_up(o + (size_t)p.M * p.nseg * sizeof(int32_t));
  p.total = o;
  return p;
}

int check_head(int64_t R, int32_t B, int64_t d, int64_t vocab, int32_t dtype) {
  if (!dtype_ok(dtype)) return DFLASH_ERR_DTYPE;
  if (R < 1 || B < 1 || d <= 0 || d % 8 != 0 || d > 16384 || vocab <= 0 || vocab % 4 != 0 ||
      vocab >= ((int64_t)1 << 30) || R * (B - 1) > INT32_MAX / 2)
    return DFLASH_ERR_SHAPE;
  return DFLASH_OK;
}
}  // namespace

extern "C" {

size_t dflash_draft_head_ws_bytes(int64_t R, int32_t B, int64_t d, int64_t vocab, int32_t dtype) {
  if (check_head(R, B, d, vocab, dtype) != DFLASH_OK || B == 1) return 0;
  return plan_head(R, B, d, vocab, elem_bytes(dtype)).total;
}

int dflash_draft_head(const void* h, int64_t R, int32_t B, int64_t d, const void* gamma_f, float eps,
                      const void* w_lm, int64_t vocab, int32_t dtype, int32_t* token_ids, float* max_logit,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = check_head(R, B, d, vocab, dtype);
  if (st) return st;
  if (!(eps >= 0.f)) return DFLASH_ERR_SHAPE;
  if (B == 1) return DFLASH_OK;
  if (!h || !gamma_f || !w_lm || !token_ids || !ws) return DFLASH_ERR_ARG;
  if (!aligned16(h) || !aligned16(gamma_f) || !aligned16(w_lm) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(token_ids) & 3) || (reinterpret_cast<uintptr_t>(max_logit) & 3))
    return DFLASH_ERR_ARG;
  const size_t eb = elem_bytes(dtype);
  HeadPlan p = plan_head(R, B, d, vocab, eb);
  if (ws_bytes < p.total) return DFLASH_ERR_WORKSPACE;
  char* w = static_cast<char*>(ws);
  void* x = w + p.off_x;
  GemmJob j = p.j;
  j.x0 = x;
  j.w = w_lm;
  j.part = reinterpret_cast<float*>(w + p.off_part);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = staged(DFLASH_STAGE_HEAD_NORM, s, true,
                        [&] { return launch_head_norm(dtype, h, p.M, B, d, gamma_f, eps, x, s); });
  if (e == hipSuccess) e = staged(DFLASH_STAGE_HEAD_GEMM, s, true, [&] { return run_gemms(dtype, {j}, s); });
  if (e == hipSuccess)
    e = staged(DFLASH_STAGE_HEAD_ARGMAX, s, true, [&] {
      return launch_head_argmax(j.part, j.plan.splits, p.M, vocab, reinterpret_cast<float*>(w + p.off_val),
                                reinterpret_cast<int32_t*>(w + p.off_idx), token_ids, max_logit, s);
    });
  return hip_status(e);
}

int dflash_accept(const int32_t* draft_ids, const int32_t* posterior, int64_t R, int32_t B, int32_t* acc,
                  int32_t* next_rows, int32_t* next_anchor, void* stream) {
  if (R < 0 || R >= ((int64_t)1 << 31) || B < 1) return DFLASH_ERR_SHAPE;
  auto misaligned = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3) != 0; };
  if (misaligned(draft_ids) || misaligned(posterior) || misaligned(acc) || misaligned(next_rows) ||
      misaligned(next_anchor))
    return DFLASH_ERR_ARG;
  if (R == 0) return DFLASH_OK;
  if (!posterior || !acc || (B > 1 && !draft_ids)) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(staged(DFLASH_STAGE_ACCEPT, s, true, [&] {
    return launch_accept(draft_ids, posterior, R, B, acc, next_rows, next_anchor, s);
  }));
}

int dflash_timing_enable(int on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = on != 0;
  return DFLASH_OK;
}

// Collects every pending pair (waiting for its end event), then reports.
int dflash_timing_read(int32_t stage, int64_t* launches, double* total_ms) {
  if (stage < 0 || stage >= DFLASH_STAGE_COUNT || !launches || !total_ms) return DFLASH_ERR_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  int st = DFLASH_OK;
  for (const auto& r : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = DFLASH_ERR_HIP;
    } else {
      t.launches[r.stage] += 1;
      t.ms[r.stage] += ms;
    }
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  *launches = t.launches[stage];
  *total_ms = t.ms[stage];
  return st;
}

int dflash_gemm_plan(int64_t M, int64_t N, int64_t K, int32_t dtype, int32_t* out) {
  if (!out) return DFLASH_ERR_ARG;
  if (!dtype_ok(dtype)) return DFLASH_ERR_DTYPE;
  if (M < 1 || N < 1 || K < 1 || M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30) || K > ((int64_t)1 << 30))
    return DFLASH_ERR_SHAPE;
  const size_t eb = elem_bytes(dtype);
  const GemmJob j = make_job(nullptr, M, nullptr, 0, nullptr, N, K, eb);
  const SkinnyPlan& p = j.plan;
  int32_t kind = DFLASH_GEMM_LDS;
  if (p.tile) kind = DFLASH_GEMM_TILE;
  else if (p.resident) kind = DFLASH_GEMM_RESIDENT;
  else if (p.fullk) kind = DFLASH_GEMM_FULLK;
  else if (p.stream) kind = DFLASH_GEMM_STREAM;
  else if (p.slab) kind = DFLASH_GEMM_SLAB;
  else if (p.wide) kind = DFLASH_GEMM_WIDE;
  out[0] = kind;
  out[1] = p.splits;
  out[2] = p.k_chunk;
  out[3] = p.n_tiles;
  out[4] = p.tile ? p.tile_bn : 0;
  out[5] = p.tile ? 0 : (int32_t)rows_per_problem(K, eb);
  return DFLASH_OK;
}

int dflash_attn_plan(const int64_t* keys, int32_t R, int32_t n_kv, int64_t chunk_cap, int32_t cache_dtype,
                     int64_t* out) {
  if (!keys || !out) return DFLASH_ERR_ARG;
  if (!cache_dtype_ok(cache_dtype)) return DFLASH_ERR_DTYPE;
  if (R < 1 || R > DFLASH_MAX_SEQS || n_kv < 1 || chunk_cap < 64) return DFLASH_ERR_SHAPE;
  std::vector<int64_t> k(keys, keys + R);
  for (int64_t x : k)
    if (x < 1 || x > ((int64_t)1 << 40)) return DFLASH_ERR_SHAPE;
  const AttnSplit sp =
      plan_attn_split(k, n_kv, std::min<int64_t>(chunk_cap, (int64_t)1 << 30), cache_dtype == DFLASH_FP8_E4M3);
  out[0] = sp.chunk;
  out[1] = sp.items;
  out[2] = sp.nst;
  return DFLASH_OK;
}

int dflash_cache_device_begin(dflash_cache* c, int32_t* d_len, void* stream) {
  if (!c || !d_len || (reinterpret_cast<uintptr_t>(d_len) & 3) || c->dev) return DFLASH_ERR_ARG;
  if (c->desc.ring) return DFLASH_ERR_SHAPE;
  LenArgs a{};
  a.d_len = d_len;
  a.R = c->desc.n_seqs;
  a.set = 1;
  for (int r = 0; r < a.R; ++r) a.value[r] = c->len[r];
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = staged(DFLASH_STAGE_PAGE_TABLE, s, true, [&] { return launch_len_update(a, s); });
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  c->d_len = d_len;
  c->dev = true;
  return DFLASH_OK;
}

int dflash_cache_device_reset(dflash_cache* c, const int32_t* host_len, void* stream) {
  if (!c || !c->dev || !host_len) return DFLASH_ERR_ARG;
  for (int r = 0; r < c->desc.n_seqs; ++r)
    if (host_len[r] < 0 || host_len[r] > c->len[r]) return DFLASH_ERR_RANGE;
  LenArgs a{};
  a.d_len = c->d_len;
  a.R = c->desc.n_seqs;
  a.set = 1;
  for (int r = 0; r < a.R; ++r) a.value[r] = host_len[r];
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = staged(DFLASH_STAGE_PAGE_TABLE, s, true, [&] { return launch_len_update(a, s); });
  return hip_status(e);
}

int dflash_cache_crop_tail_dev(dflash_cache* c, int32_t drop, void* stream) {
  if (!c || !c->dev) return DFLASH_ERR_ARG;
  if (drop < 0) return DFLASH_ERR_RANGE;
  LenArgs a{};
  a.d_len = c->d_len;
  a.R = c->desc.n_seqs;
  a.delta = -drop;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = staged(DFLASH_STAGE_PAGE_TABLE, s, true, [&] { return launch_len_update(a, s); });
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  // the bounds drop as the true lengths do; pages past the bounds hold no row
  std::vector<int32_t> bound(c->desc.n_seqs);
  for (int r = 0; r < c->desc.n_seqs; ++r) bound[r] = std::max(0, c->len[r] - drop);
  crop_host(c, bound.data());
  return DFLASH_OK;
}

int dflash_cache_device_end(dflash_cache* c, void* stream) {
  if (!c || !c->dev) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> v(c->desc.n_seqs);
  if (hipStreamSynchronize(s) != hipSuccess ||
      hipMemcpy(v.data(), c->d_len, v.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return DFLASH_ERR_HIP;
  for (int r = 0; r < c->desc.n_seqs; ++r)
    if (v[r] < 0 || v[r] > c->len[r]) return DFLASH_ERR_RANGE;
  crop_host(c, v.data());
  c->dev = false;
  c->d_len = nullptr;
  return DFLASH_OK;
}

int dflash_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0) return DFLASH_ERR_SHAPE;
  if (bytes == 0) return DFLASH_OK;
  if (!src || !aligned16(src) || (reinterpret_cast<uintptr_t>(sink) & 3)) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(
      staged(DFLASH_STAGE_STREAM_READ, s, bytes >= 16, [&] { return launch_stream_read(src, bytes, sink, s); }));
}

int dflash_mfma_peak(int32_t iters, int64_t workgroups, float* sink, void* stream) {
  if (iters < 1 || iters > (1 << 24) || workgroups < 1 || workgroups > (1 << 20)) return DFLASH_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(sink) & 3) return DFLASH_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(
      staged(DFLASH_STAGE_MFMA_PEAK, s, true, [&] { return launch_mfma_peak(iters, workgroups, sink, s); }));
}

int dflash_attn_sync_timeouts(uint32_t* count) {
  if (!count) return DFLASH_ERR_ARG;
  uint32_t bf = 0, f8 = 0;
  hipError_t e = attn_sync_timeouts(&bf);
  if (e == hipSuccess) e = attn_fp8_sync_timeouts(&f8);
  if (e != hipSuccess) return DFLASH_ERR_HIP;
  *count = bf + f8;
  return DFLASH_OK;
}

int dflash_attn_force_merge_spread(int32_t on) {
  if (on != 0 && on != 1) return DFLASH_ERR_ARG;
  g_merge_spread.store(on);
  return DFLASH_OK;
}

int dflash_attn_set_spin_limit(int32_t polls) {
  if (polls < 0 || polls > kAttnSpinLimit) return DFLASH_ERR_ARG;
  g_spin_limit.store(polls);
  return DFLASH_OK;
}

int dflash_attn_force_chunk(int64_t chunk) {
  if (chunk != 0 && (chunk < 64 || chunk % 64 != 0 || chunk > ((int64_t)1 << 30))) return DFLASH_ERR_SHAPE;
  g_forced_chunk.store(chunk);
  return DFLASH_OK;
}

int dflash_timing_reset(void) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (const auto& r : t.pending) {
    (void)hipEventSynchronize(r.b);
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
  for (int i = 0; i < DFLASH_STAGE_COUNT; ++i) {
    t.launches[i] = 0;
    t.ms[i] = 0.0;
  }
  return DFLASH_OK;
}

}  // extern "C"
