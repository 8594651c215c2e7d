// api.cpp -- the extern "C" boundary of libmxfp4.so: argument checks, plan
// selection, workspace carving and launches.  Every check happens before
// anything is enqueued, so an error other than MXFP4_EHIP leaves the stream
// untouched.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "mxfp4.h"
#include "mx_internal.hpp"

// ---------------------------------------------------- allocation-free entry
// Device scratch of mxfp4_gemm_noalloc: a fixed array in the library's own
// device code, one copy per GPU, held until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): each device's copy is looked up once with
// hipGetSymbolAddress (device_scratch below), and that pointer is what the
// kernels get.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// the same signature as fail(), for checks that must not touch the message
int quiet(int code, const char*, ...) { return code; }

int ok() {
  g_err[0] = '\0';
  return MXFP4_OK;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int hip_fail(hipError_t e, const char* what) {
  return fail(MXFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

mx::Plan to_internal(const mxfp4_plan& p) {
  mx::Plan q;
  q.mode = p.mode;
  q.mbw = p.m_blocks;
  q.ntw = p.n_tiles_per_wave;
  q.wn = p.waves_n;
  q.wk = p.waves_k;
  q.ksw = p.k_steps_per_wave;
  q.split = p.split_k;
  q.reduce = p.split_k > 1 ? p.split_reduce : mx::kReduceKernel;
  return q;
}

mxfp4_plan make_plan(int mode, int mbw, int ntw, int wn, int wk, int ksw, int split,
                     int reduce = MXFP4_REDUCE_KERNEL) {
  mxfp4_plan p;
  p.split_reduce = reduce;
  p.mode = mode;
  p.m_blocks = mbw;
  p.n_tiles_per_wave = ntw;
  p.waves_n = wn;
  p.waves_k = wk;
  p.k_steps_per_wave = ksw;
  p.split_k = split;
  return p;
}

// `call`: the shape of a GEMM call, where M or N may be 0 (an empty call,
// which returns before this check); a plan needs both >= 1.
int check_gemm_shape(int M, int N, int K, bool call = false) {
  if (K < 32 || K % 32 != 0) return fail(MXFP4_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  const int lo = call ? 0 : 1;
  if (M < lo) return fail(MXFP4_EINVAL, "M must be >= %d (got %d)", lo, M);
  if (N < lo) return fail(MXFP4_EINVAL, "N must be >= %d (got %d)", lo, N);
  if ((long long)M * K > (1LL << 40) || (long long)N * K > (1LL << 40) || (long long)M * N > (1LL << 40))
    return fail(MXFP4_EINVAL, "shape too large");
  return MXFP4_OK;
}

// An empty call: `rows` (M, or N where B's rows are the operand) or `cols`
// (N of a product; 0 = none) is 0, the others are valid and K is a positive
// multiple of 32.  There is nothing to read or write: the entry points
// return success before looking at any pointer or launching anything.
bool empty_call(int rows, int cols, int K) {
  return rows >= 0 && cols >= 0 && (rows == 0 || cols == 0) && K >= 32 && K % 32 == 0;
}

// Tile width of a tiled plan: waves_n == 2 selects 256 x 128 tiles (four
// wavefronts), any other value 256 x 256 (eight).
int tiled_width(const mxfp4_plan& p) { return p.waves_n == 2 ? 128 : 256; }

// Stream-mode plan rules: four wavefronts along N, k_steps_per_wave is the
// workgroup's K range in steps (a multiple of 4), and split_k the number of
// workgroups that cover K with it.
int check_stream_plan(const mxfp4_plan& p, int M, int N, int K, int (*bad)(int, const char*, ...)) {
  if (!mx::stream_kernel_available(p.m_blocks, p.n_tiles_per_wave))
    return bad(MXFP4_ENOTSUP, "MXFP4_MODE_STREAM has no kernel for m_blocks=%d n_tiles_per_wave=%d",
               p.m_blocks, p.n_tiles_per_wave);
  if (p.waves_n != 4 || p.waves_k != 1)
    return bad(MXFP4_EINVAL, "MXFP4_MODE_STREAM runs four wavefronts along N (waves_n = 4, waves_k = 1)");
  if (K > mx::kStreamMaxK)
    return bad(MXFP4_EINVAL, "MXFP4_MODE_STREAM supports K <= %d (got %d)", mx::kStreamMaxK, K);
  const int KS = (int)(((long long)K + 127) / 128), KG = (KS + 3) / 4;
  if (p.k_steps_per_wave < 4 || p.k_steps_per_wave % 4 != 0 || p.k_steps_per_wave / 4 > KG)
    return bad(MXFP4_EINVAL,
               "MXFP4_MODE_STREAM: k_steps_per_wave is the workgroup's K steps, a multiple of 4 "
               "in [4, %d] (got %d)", 4 * KG, p.k_steps_per_wave);
  const int chunks = p.k_steps_per_wave / 4;
  const int split = (KG + chunks - 1) / chunks;
  if (p.split_k != split)
    return bad(MXFP4_EINVAL, "MXFP4_MODE_STREAM: %d steps per workgroup need split_k = %d (got %d)",
               p.k_steps_per_wave, split, p.split_k);
  if (split > 1 && p.split_reduce != MXFP4_REDUCE_KERNEL)
    return bad(MXFP4_EINVAL, "MXFP4_MODE_STREAM sums split partials with the reduce kernel only");
  const mx::StreamGeom g = mx::stream_geometry(p.m_blocks, p.n_tiles_per_wave, p.k_steps_per_wave, M, N, K);
  if (g.grid * g.threads > 0xFFFFFFFFLL)
    return bad(MXFP4_EINVAL, "grid too large (%lld workgroups of %d threads)", g.grid, g.threads);
  if (split > 1) {
    const long long n = (N % 4 == 0) ? (long long)M * (N / 4) : (long long)M * N;
    if (n > 0xFFFFFFFFLL - 63) return bad(MXFP4_EINVAL, "split-K reduce grid too large (%lld threads)", n);
  }
  return MXFP4_OK;
}

// Checks a plan against a shape; `mode_matters` is false for the prequant
// entry point, where the mode only selects the tiled or stream kernel or not.
int check_plan(const mxfp4_plan& p, int M, int N, int K, bool mode_matters,
               bool report = true) {
  int (*const bad)(int, const char*, ...) = report ? fail : quiet;
  if (mode_matters && p.mode != MXFP4_MODE_FUSED && p.mode != MXFP4_MODE_PREQUANT &&
      p.mode != MXFP4_MODE_TILED && p.mode != MXFP4_MODE_STREAM)
    return bad(MXFP4_EINVAL,
               "plan.mode must be MXFP4_MODE_FUSED, _PREQUANT, _TILED or _STREAM (got %d)", p.mode);
  if (p.mode == MXFP4_MODE_STREAM) return check_stream_plan(p, M, N, K, bad);
  if (p.mode == MXFP4_MODE_TILED) {
    // waves_n picks the tile width, split_k the workgroups along K (with
    // split_reduce); the other fields are not used
    if (K > mx::kTiledMaxK)
      return bad(MXFP4_EINVAL, "MXFP4_MODE_TILED supports K <= %d (got %d)", mx::kTiledMaxK, K);
    const int KS = (int)(((long long)K + 127) / 128), KG = (KS + 3) / 4;
    if (p.split_k < 1 || p.split_k > KG)
      return bad(MXFP4_EINVAL,
                 "MXFP4_MODE_TILED: split_k must be in [1, %d] (whole groups of four K steps per "
                 "workgroup; got %d)", KG, p.split_k);
    const mx::TiledGeom t = mx::tiled_geometry(M, N, K, tiled_width(p), p.split_k);
    if ((long long)(p.split_k - 1) * t.sps >= KS)
      return bad(MXFP4_EINVAL,
                 "MXFP4_MODE_TILED: split_k = %d leaves a workgroup without K steps (%d steps in "
                 "ranges of %d)", p.split_k, KS, t.sps);
    if (p.split_k > 1 && p.split_reduce != MXFP4_REDUCE_KERNEL)
      return bad(MXFP4_EINVAL, "MXFP4_MODE_TILED sums split partials with the reduce kernel only");
    if (t.grid * t.threads > 0xFFFFFFFFLL)
      return bad(MXFP4_EINVAL, "grid too large (%lld workgroups of %d threads)", t.grid, t.threads);
    if (p.split_k > 1) {
      const long long n = (N % 4 == 0) ? (long long)M * (N / 4) : (long long)M * N;
      if (n > 0xFFFFFFFFLL - 63) return bad(MXFP4_EINVAL, "split-K reduce grid too large (%lld threads)", n);
    }
    return MXFP4_OK;
  }
  if (p.m_blocks < 1 || p.n_tiles_per_wave < 1 || p.waves_n < 1 || p.waves_k < 1 ||
      p.k_steps_per_wave < 1 || p.split_k < 1)
    return bad(MXFP4_EINVAL, "plan fields must all be >= 1");
  if (p.split_reduce != MXFP4_REDUCE_KERNEL && p.split_reduce != MXFP4_REDUCE_LAST_WG &&
      p.split_reduce != MXFP4_REDUCE_ATOMIC)
    return bad(MXFP4_EINVAL,
                "plan.split_reduce must be MXFP4_REDUCE_KERNEL, _LAST_WG or _ATOMIC (got %d)",
                p.split_reduce);
  if (p.split_k > mx::kMaxLastWgSplit && p.split_reduce == MXFP4_REDUCE_LAST_WG)
    return bad(MXFP4_EINVAL, "split_reduce LAST_WG supports split_k <= %d (got %d)", mx::kMaxLastWgSplit,
                p.split_k);
  const int mode = mode_matters ? p.mode : MXFP4_MODE_PREQUANT;
  if (!mx::gemm_kernel_available(mode, p.m_blocks, p.n_tiles_per_wave, p.k_steps_per_wave))
    return bad(MXFP4_ENOTSUP,
                "no kernel for m_blocks=%d n_tiles_per_wave=%d k_steps_per_wave=%d in this library",
                p.m_blocks, p.n_tiles_per_wave, p.k_steps_per_wave);
  // each factor is bounded before any product is formed, so absurd field
  // values cannot overflow the arithmetic below
  const long long waves = (long long)p.waves_n * p.waves_k;
  if (waves > mx::kMaxThreads / 64)
    return bad(MXFP4_EINVAL, "plan has %lld wavefronts per workgroup (max %d)", waves,
                mx::kMaxThreads / 64);
  const int KS = (int)(((long long)K + 127) / 128);
  if (p.split_k > KS || (long long)p.split_k * p.waves_k * p.k_steps_per_wave != KS)
    return bad(MXFP4_EINVAL, "plan covers %lld K steps, shape has %d (split_k*waves_k*k_steps_per_wave must equal ceil(K/128))",
                (long long)p.split_k * p.waves_k * p.k_steps_per_wave, KS);
  mx::Plan q = to_internal(p);
  q.mode = mode;
  const mx::GemmGeom g = mx::gemm_geometry(q, M, N, K);
  if (g.lds_total > (size_t)mx::kMaxLds)
    return bad(MXFP4_EINVAL, "plan needs %zu bytes of LDS (max %d)", g.lds_total, mx::kMaxLds);
  // a dispatch holds at most 2^32 - 1 work-items
  const long long blocks = 8LL * (((long long)g.ngroups * p.split_k + 7) / 8) * g.mgroups;
  if (blocks * g.threads > 0xFFFFFFFFLL)
    return bad(MXFP4_EINVAL, "grid too large (%lld workgroups of %d threads)", blocks, g.threads);
  if (p.split_k > 1 && p.split_reduce == MXFP4_REDUCE_KERNEL) {
    const long long n = (N % 4 == 0) ? (long long)M * (N / 4) : (long long)M * N;
    if (n > 0xFFFFFFFFLL - 63) return bad(MXFP4_EINVAL, "split-K reduce grid too large (%lld threads)", n);
  }
  return MXFP4_OK;
}

// Workspace layout: [tile counters][fp32 partials or accumulator][MX-packed A],
// each part rounded up to 256 bytes.  The counters, and the accumulator of
// the atomic reduce, must start at zero and are left zero by every call.
struct WsLayout {
  size_t counters, partials, a;  // byte sizes
  bool zero_partials;            // the partials part is the atomic accumulator
  size_t part_off() const { return counters; }
  size_t a_off() const { return counters + partials; }
  size_t zero_bytes() const { return counters + (zero_partials ? partials : 0); }
  size_t total() const { return counters + partials + a; }
};

WsLayout ws_layout(const mxfp4_plan& p, int M, int N, int K, bool prequant_entry) {
  WsLayout w = {0, 0, 0, false};
  if (p.mode == MXFP4_MODE_TILED) {
    if (p.split_k > 1) w.partials = round_up((size_t)p.split_k * M * N * 4, 256);
    if (!prequant_entry) w.a = round_up(mxfp4_packed_bytes(M, K), 256);
    return w;
  }
  if (p.mode == MXFP4_MODE_STREAM) {
    if (p.split_k > 1) w.partials = round_up((size_t)p.split_k * M * N * 4, 256);
    if (!prequant_entry) w.a = round_up(mxfp4_packed_bytes(M, K), 256);
    return w;
  }
  const bool split = p.split_k > 1;
  if (split && p.split_reduce != MXFP4_REDUCE_KERNEL) {
    const mx::GemmGeom g = mx::gemm_geometry(to_internal(p), M, N, K);
    w.counters = round_up((size_t)g.mgroups * g.ngroups * 4, 256);
  }
  if (split) {
    const size_t planes = p.split_reduce == MXFP4_REDUCE_ATOMIC ? 1 : (size_t)p.split_k;
    w.partials = round_up(planes * M * N * 4, 256);
    w.zero_partials = p.split_reduce == MXFP4_REDUCE_ATOMIC;
  }
  if (!prequant_entry && p.mode == MXFP4_MODE_PREQUANT)
    w.a = round_up(mxfp4_packed_bytes(M, K), 256);
  return w;
}

// Estimated L2-cold microseconds of a plan, a model fitted to L2-cold sweeps
// of every plan on 20 shapes (M 1..640, N 1024..8192, K 512..16384; the
// fitted picks are within 7 % of the best plan on each): each workgroup
// streams its A rows (bf16 when fused, fp4 + scales when pre-quantized) and
// B columns (fp4 + scales) for its K range at up to 100 GB/s per CU, less
// with fewer than eight wavefronts (fused mode: whole 16-row blocks of bf16
// A, whatever M), and in fused mode quantizes its A rows
// (about 2 us per 64 Ki elements); each further 256 workgroups is another
// round; a split-K adds the reduce launch, its partials and a little per
// slice; pre-quantized A adds the quantizer launch and its traffic; a small
// cost per extra K wavefront.
double plan_cost(const mxfp4_plan& p, int M, int N, int K) {
  const long long MT = ((long long)M + 15) / 16, NT = ((long long)N + 15) / 16;
  const long long cols_wg = (long long)p.waves_n * p.n_tiles_per_wave;
  const long long wgs = ((MT + p.m_blocks - 1) / p.m_blocks) * ((NT + cols_wg - 1) / cols_wg) *
                        p.split_k;
  const double rounds = ceil(wgs / 256.0);
  const double rows = fmin(16.0 * p.m_blocks, (double)M);
  const double cols = fmin(16.0 * cols_wg, (double)N);
  const double kel = 128.0 * p.waves_k * p.k_steps_per_wave;
  const bool fused = p.mode == MXFP4_MODE_FUSED;
  const double a_bytes = fused ? 2.0 : 17.0 / 32.0;  // per element
  // fused mode loads whole 16-row blocks of A (rows past M repeat earlier
  // rows, so the load count is fixed), and each load costs its issue
  const double a_rows = fused ? 16.0 * p.m_blocks : rows;
  const double bytes = a_rows * kel * a_bytes + cols * kel * 17.0 / 32.0;
  const int waves = p.waves_n * p.waves_k;
  const double rate = 100000.0 * fmin(1.0, pow(waves / 8.0, 0.75));  // bytes per us
  double t = rounds * bytes / rate;
  if (fused) t += 2.0 * rounds * rows * kel / 65536.0;
  if (p.split_k > 1) t += 2.0 + (double)p.split_k * M * N * 4.0 / 5.0e6 + 0.05 * p.split_k;
  if (!fused) t += 2.65 + (double)M * K * 2.5 / 5.0e6;
  t += 0.1 * (p.waves_k - 1);
  return t;
}

// Estimated L2-cold microseconds per call of the tiled mode through
// mxfp4_gemm, fitted to event timings of 39 runs (18 shapes from
// 256x4096x4096 to 3072x3072x1024 at both tile widths, and 1024x8192x8192,
// 4096^3 and 8192^3; within 10 % on all but one, 14 %): the launch floor,
// the quantizer's launch and its A traffic at 5.7 TB/s (its measured rate),
// then per round of up to 256 tiles 0.55 us plus, per 128-K step, 0.61 to
// 1.03 us for a 256 x 256 tile (the slower when more CUs run at once, as the
// clock drops) and kHalfTileStep of that for a 256 x 128 one.  A split of K
// over workgroups runs split times as many workgroups of a split-th of the
// steps (whole groups of four), then the reduce launch: 4 us plus the fp32
// partials written and read and C at 7 TB/s (fitted to 360 timings of
// split and unsplit tiled plans on 30 shapes with M 256..1024: picks a mean
// 1.0 % and at most 9 % slower than the fastest tiled plan of each shape).
constexpr double kHalfTileStep = 0.608;
double tiled_cost(int M, int N, int K, int width, int split) {
  const double tiles = ceil(M / 256.0) * ceil(N / (double)width);
  const double tasks = tiles * split;
  const double rounds = ceil(tasks / 256.0);
  double step_us = 0.613 + 0.413 * fmin(1.0, tasks / 256.0);
  if (width != 256) step_us *= kHalfTileStep;
  const double ks = ceil(K / 128.0);
  const double sps = fmin(ks, 4.0 * ceil(ceil(ks / split) / 4.0));
  double t = 10.48 + (double)M * K * 2.5 / 5.7e6 + rounds * (step_us * sps + 0.55);
  if (split > 1) t += 4.0 + ((double)split * M * N * 8.0 + 2.0 * M * N) / 7.0e6;
  return t;
}

// plan_cost is relative: it omits the launch floor and, on shapes with
// hundreds of thousands of products per CU, the issue rate of the
// 16x16x128 kernels, which reach 0.6 to 0.85 PFLOP/s there (measured on
// nine shapes from 512x4096x4096 to 4096^3; 0.7 is used).  Against the
// tiled mode's absolute estimate they count both.
double absolute_cost(const mxfp4_plan& p, int M, int N, int K) {
  return 6.3 + fmax(plan_cost(p, M, N, K), 2.0 * M * N * (double)K / 0.7e9);
}

// The valid plan (reduce kernel for split-K) of least plan_cost; fused before
// pre-quantized, so ties keep the single-launch plan.  Shapes with M >= 256
// and at least 16 tiles of 256 x 256 also weigh the tiled mode.
mxfp4_plan model_plan(int M, int N, int K) {
  static const int ksw_opts[] = {1, 2, 3, 4, 6, 7, 8, 12, 14, 16};
  static const int wk_opts[] = {1, 2, 3, 4, 8};
  const long long KS = ((long long)K + 127) / 128;
  const long long MT = ((long long)M + 15) / 16, NT = ((long long)N + 15) / 16;
  mxfp4_plan best = make_plan(MXFP4_MODE_FUSED, 1, 1, 1, 1, 1, (int)KS);
  double best_t = 1e300;
  for (int mode : {MXFP4_MODE_FUSED, MXFP4_MODE_PREQUANT})
    for (int mbw : {1, 2, 4}) {
      if (mbw > 1 && mbw > MT) continue;
      for (int ntw : {1, 2})
        for (int wn = 1; wn <= 8; ++wn) {
          if ((long long)wn * ntw > NT) continue;
          for (int wk : wk_opts) {
            if (wn * wk > mx::kMaxThreads / 64) continue;
            for (int ksw : ksw_opts) {
              if (KS % ((long long)wk * ksw)) continue;
              const mxfp4_plan p =
                  make_plan(mode, mbw, ntw, wn, wk, ksw, (int)(KS / ((long long)wk * ksw)));
              if (check_plan(p, M, N, K, true, false) != MXFP4_OK) continue;
              const double t = plan_cost(p, M, N, K);
              if (t < best_t) {
                best_t = t;
                best = p;
              }
            }
          }
        }
    }
  if (M >= 256 && ceil(M / 256.0) * ceil(N / 256.0) >= 16) {
    double best_abs = absolute_cost(best, M, N, K);
    mxfp4_plan pick = best;
    for (int wn : {4, 2})  // 256 x 256 tiles, then 256 x 128
      for (int split : {1, 2, 3, 4, 6, 8}) {
        const mxfp4_plan tiled = make_plan(MXFP4_MODE_TILED, 1, 1, wn, 1, 1, split);
        const double t = tiled_cost(M, N, K, tiled_width(tiled), split);
        if (check_plan(tiled, M, N, K, true, false) == MXFP4_OK && t < best_abs) {
          best_abs = t;
          pick = tiled;
        }
      }
    return pick;
  }
  return best;
}

// model_plan is a search over about 4,000 candidates; mxfp4_gemm without a plan
// asks for it on every call, so the last few shapes' picks are kept.
mxfp4_plan cached_model_plan(int M, int N, int K) {
  struct Entry {
    int M, N, K;
    mxfp4_plan p;
  };
  constexpr int kEntries = 64;
  static std::mutex mu;
  static Entry cache[kEntries];
  static int used = 0, next = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].M == M && cache[i].N == N && cache[i].K == K) return cache[i].p;
  }
  const mxfp4_plan p = model_plan(M, N, K);
  std::lock_guard<std::mutex> lock(mu);
  cache[next] = Entry{M, N, K, p};
  next = (next + 1) % kEntries;
  if (used < kEntries) ++used;
  return p;
}

// Smallest split of K over workgroups that gives the stream kernel 192
// workgroups or more (all of K when fewer chunks are left).
int stream_split(int M, int N, int K, int mbw, int ntw) {
  const long long MT = ((long long)M + 15) / 16, NT = ((long long)N + 15) / 16;
  const int KG = (int)((((long long)K + 127) / 128 + 3) / 4);
  const long long mg = (MT + mbw - 1) / mbw, ng = (NT + 4 * ntw - 1) / (4 * ntw);
  int split = 1;
  while (ng * mg * split < 192 && split < KG) ++split;
  return split;
}

// The stream plan: the row blocks of up to 64 rows in one workgroup (one
// block or two for M <= 32), fewer (halving) while that would need K split
// over workgroups and K < 20480 (a split adds the reduce launch and fp32
// partials, which only a long K repays), two 16-column tiles per wavefront
// with 65 rows or more, four row blocks, N x K >= 50M and no split, and the
// smallest split that gives 192 workgroups.  On the 225 training shapes of
// the rule below this pick was a mean 0.3 % (at most 6 %) slower than the
// fastest of the six tilings with one, two or four row blocks and one or two
// tiles per wavefront; on ten held-out shapes with M >= 112 where it takes
// two tiles per wavefront, 0.90-1.06 of the time with one.
mxfp4_plan stream_plan(int M, int N, int K) {
  const int MT = (M + 15) / 16, KS = (int)(((long long)K + 127) / 128), KG = (KS + 3) / 4;
  int mbw = MT <= 2 ? MT : 4;
  while (mbw > 1 && K < 20480 && stream_split(M, N, K, mbw, 1) > 1) mbw /= 2;
  const int ntw = (MT >= 5 && mbw == 4 && (long long)N * K >= 50LL * 1000 * 1000 &&
                   stream_split(M, N, K, 4, 2) == 1)
                      ? 2
                      : 1;
  const int split = stream_split(M, N, K, mbw, ntw);
  const int chunks = (KG + split - 1) / split;
  return make_plan(MXFP4_MODE_STREAM, mbw, ntw, 4, 1, 4 * chunks, (KG + chunks - 1) / chunks);
}

// Stream mode where it measured faster.  Rules fitted on 225 training shapes
// (M 1..255 against 15 sizes of B, N x K 17M..268M, K >= 4096), timed
// L2-cold against the cost model's or the small-M rule's pick, then checked
// on two sets of 110 held-out shapes (M 3..250, twenty other sizes of B).
// Time of the stream plan over the other pick on the training shapes: with
// M >= 96, 0.58-0.94 (20 shapes); with M 17..95 where its workgroups keep
// two or four row blocks and N >= 4096 (M >= 48), N >= 7168, or K >= 8192
// and N x K >= 100M, 0.65-0.94 (29); with M <= 16 against a large B with
// long K and no split of K unless K >= 20480, 0.88-1.00 (13).  Left out:
// one row block below M = 96 (B is read once per 16 rows; 1.06-1.09 on
// four held-out shapes), a split with K < 20480 at M <= 16 (1.20 at
// 14x8192x16384), and smaller B at M <= 16 (up to 1.46).  M 256..512 with
// N x K <= 70M and N <= 8192 (M = 256), N <= 6144 (up to M = 320), or N <=
// 4096 and N x K <= 40M: 0.51-0.98 against the tiled or other pick on 25
// shapes, 0.74-0.89 against the fastest tiled plan (nontemporal copies, any
// split) on seven; beyond those bounds the tiled mode won (by 5 % at
// 384/512 x 4096 x 11008, 12 % at 320 x 7168 x 7168, 20-50 % at N >= 11008).
bool use_stream(int M, int N, int K) {
  const long long nk = (long long)N * K;
  if (M > 512 || K < 4096 || nk < 16LL * 1000 * 1000) return false;
  if (M > 255) {
    if (nk > 70LL * 1000 * 1000 || N < 2048) return false;
    if (M <= 256) return N <= 8192;
    if (M <= 320) return N <= 6144;
    return N <= 4096 && nk <= 40LL * 1000 * 1000;
  }
  const mxfp4_plan p = stream_plan(M, N, K);
  if (M <= 16)
    return K >= 8192 && (p.split_k == 1 || K >= 20480) &&
           ((nk >= 150LL * 1000 * 1000 && M >= 8) || (nk >= 100LL * 1000 * 1000 && M >= 13));
  if (M >= 96) return N >= 2048;
  if (p.m_blocks == 1) return false;
  if (K >= 8192 && nk >= 100LL * 1000 * 1000) return true;
  return N >= (M >= 48 ? 4096 : 7168);
}

// Small M against a B with long K: the fused kernel with one row block and
// eight wavefronts along N, 16 (or 14, 12, 8) steps per wavefront and K
// split over workgroups.  Measured L2-cold against the cost model's pick: on
// 54 shapes with M 1..16 and N x K 59M..268M, 1.01-1.31x as fast on 28 of
// the 30 shapes with K >= 8192 and N x K >= 100M (0.99x on two), losing by
// up to 12 % below those sizes; on the 225 shapes of the stream rule, where
// that rule leaves M <= 32 with N <= 4096, 1.03-1.13x as fast with M 17..32,
// K >= 8192 and N x K >= 30M, and 1.00-1.14x with M <= 16 and K >= 14336
// (0.996x on one of 18), but 0.93-0.98x with M <= 16 and K = 8192.
mxfp4_plan small_m_plan(int M, int N, int K, bool* ok) {
  const int KS = (int)(((long long)K + 127) / 128);
  const long long nk = (long long)N * K;
  *ok = false;
  const bool take = M <= 16 ? K >= 8192 && (nk >= 100LL * 1000 * 1000 || (K >= 14336 && nk >= 30LL * 1000 * 1000))
                            : M <= 32 && N <= 4096 && K >= 8192 && nk >= 30LL * 1000 * 1000;
  if (!take) return mxfp4_plan{};
  for (int ksw : {16, 14, 12, 8})
    if (KS % ksw == 0) {
      *ok = true;
      return make_plan(MXFP4_MODE_FUSED, 1, 1, 8, 1, ksw, KS / ksw, MXFP4_REDUCE_KERNEL);
    }
  return mxfp4_plan{};
}

// Per-shape table for the tuned shapes, the stream and small-M rules, the
// cost model otherwise.
mxfp4_plan default_plan(int M, int N, int K) {
  struct Row {
    int M, N, K;
    mxfp4_plan p;
  };
  // Chosen by an L2-cold sweep over every valid plan on MI355X (median
  // event time per call; waves_n 1..8), then confirmed by interleaved
  // repeats against the runner-up.
  static const Row table[] = {
      {4, 2880, 512, make_plan(MXFP4_MODE_FUSED, 1, 1, 2, 1, 4, 1)},
      {32, 4096, 512, make_plan(MXFP4_MODE_FUSED, 1, 1, 2, 1, 4, 1)},
      {32, 2880, 512, make_plan(MXFP4_MODE_FUSED, 1, 1, 2, 1, 4, 1)},
      {16, 2112, 7168, make_plan(MXFP4_MODE_FUSED, 1, 1, 4, 1, 8, 7, MXFP4_REDUCE_KERNEL)},
      {64, 7168, 2048, make_plan(MXFP4_MODE_FUSED, 1, 1, 8, 1, 16, 1)},
      {256, 3072, 1536, make_plan(MXFP4_MODE_FUSED, 1, 2, 6, 1, 12, 1)},
  };
  for (const Row& r : table)
    if (r.M == M && r.N == N && r.K == K) return r.p;
  if (use_stream(M, N, K)) {
    const mxfp4_plan p = stream_plan(M, N, K);
    if (check_plan(p, M, N, K, true, false) == MXFP4_OK) return p;
  }
  bool small_m = false;
  const mxfp4_plan sp = small_m_plan(M, N, K, &small_m);
  if (small_m && check_plan(sp, M, N, K, true, false) == MXFP4_OK) return sp;
  return cached_model_plan(M, N, K);
}

int check_workspace(const void* workspace, size_t have, size_t need) {
  if (need == 0) return MXFP4_OK;
  if (!workspace) return fail(MXFP4_ENULL, "workspace is NULL but the plan needs %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MXFP4_EINVAL, "workspace must be 256-byte aligned");
  if (have < need) return fail(MXFP4_EWORKSPACE, "workspace holds %zu bytes, plan needs %zu", have, need);
  return MXFP4_OK;
}

int check_stream_ptrs(const void* p, const char* name) {
  if (!p) return fail(MXFP4_ENULL, "%s is NULL", name);
  return MXFP4_OK;
}

}  // namespace

extern "C" {

size_t mxfp4_packed_bytes(int rows, int K) {
  if (rows < 1 || K < 32 || K % 32 != 0) return 0;
  return mx::packed_dims(rows, K).total_bytes();
}

int mxfp4_pack_b(const uint8_t* b_fp4, const uint8_t* b_scale, int N, int K, void* b_packed,
                 size_t b_packed_bytes, void* stream) {
  if (empty_call(N, 1, K)) return ok();
  int rc;
  if ((rc = check_stream_ptrs(b_fp4, "b_fp4")) || (rc = check_stream_ptrs(b_scale, "b_scale")) ||
      (rc = check_stream_ptrs(b_packed, "b_packed")))
    return rc;
  if (K < 32 || K % 32 != 0) return fail(MXFP4_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (N < 0) return fail(MXFP4_EINVAL, "N must be >= 0 (got %d)", N);
  if (!aligned(b_fp4, 16) || !aligned(b_packed, 16))
    return fail(MXFP4_EINVAL, "b_fp4 and b_packed must be 16-byte aligned");
  const size_t need = mxfp4_packed_bytes(N, K);
  if (b_packed_bytes < need)
    return fail(MXFP4_ESIZE, "b_packed holds %zu bytes, layout needs %zu", b_packed_bytes, need);
  mx::launch_pack_b(b_fp4, b_scale, N, K, static_cast<uint8_t*>(b_packed),
                    static_cast<hipStream_t>(stream));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "pack_b launch");
  return ok();
}

int mxfp4_quant_a(const uint16_t* a, int M, int K, int lda, uint8_t* out_fp4, int ld_fp4,
                  uint8_t* out_scale, int ld_scale, void* stream) {
  if (empty_call(M, 1, K)) return ok();
  int rc;
  if ((rc = check_stream_ptrs(a, "a")) || (rc = check_stream_ptrs(out_fp4, "out_fp4")) ||
      (rc = check_stream_ptrs(out_scale, "out_scale")))
    return rc;
  if (K < 32 || K % 32 != 0) return fail(MXFP4_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (M < 0) return fail(MXFP4_EINVAL, "M must be >= 0 (got %d)", M);
  if (lda < K || lda % 8 != 0) return fail(MXFP4_EINVAL, "lda must be >= K and a multiple of 8 (got %d)", lda);
  if (ld_fp4 < K / 2 || ld_fp4 % 4 != 0)
    return fail(MXFP4_EINVAL, "ld_fp4 must be >= K/2 and a multiple of 4 (got %d)", ld_fp4);
  if (ld_scale < K / 32) return fail(MXFP4_EINVAL, "ld_scale must be >= K/32 (got %d)", ld_scale);
  if (!aligned(a, 16) || !aligned(out_fp4, 4))
    return fail(MXFP4_EINVAL, "a must be 16-byte and out_fp4 4-byte aligned");
  if ((long long)M * K > (1LL << 40)) return fail(MXFP4_EINVAL, "M*K too large");
  mx::launch_quant_linear(a, M, K, lda, out_fp4, ld_fp4, out_scale, ld_scale,
                          static_cast<hipStream_t>(stream));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quant_a launch");
  return ok();
}

int mxfp4_quant_a_packed(const uint16_t* a, int M, int K, int lda, void* out_packed,
                         size_t out_packed_bytes, void* stream) {
  if (empty_call(M, 1, K)) return ok();
  int rc;
  if ((rc = check_stream_ptrs(a, "a")) || (rc = check_stream_ptrs(out_packed, "out_packed")))
    return rc;
  if (K < 32 || K % 32 != 0) return fail(MXFP4_EINVAL, "K must be a positive multiple of 32 (got %d)", K);
  if (M < 0) return fail(MXFP4_EINVAL, "M must be >= 0 (got %d)", M);
  if (lda < K || lda % 8 != 0) return fail(MXFP4_EINVAL, "lda must be >= K and a multiple of 8 (got %d)", lda);
  if (!aligned(a, 16) || !aligned(out_packed, 16))
    return fail(MXFP4_EINVAL, "a and out_packed must be 16-byte aligned");
  const size_t need = mxfp4_packed_bytes(M, K);
  if (out_packed_bytes < need)
    return fail(MXFP4_ESIZE, "out_packed holds %zu bytes, layout needs %zu", out_packed_bytes, need);
  mx::launch_quant_packed(a, M, K, lda, static_cast<uint8_t*>(out_packed),
                          static_cast<hipStream_t>(stream));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "quant_a_packed launch");
  return ok();
}

int mxfp4_default_plan(int M, int N, int K, mxfp4_plan* plan) {
  if (!plan) return fail(MXFP4_ENULL, "plan is NULL");
  int rc = check_gemm_shape(M, N, K);
  if (rc) return rc;
  *plan = default_plan(M, N, K);
  return ok();
}

int mxfp4_check_plan(const mxfp4_plan* plan, int M, int N, int K) {
  if (!plan) return fail(MXFP4_ENULL, "plan is NULL");
  int rc = check_gemm_shape(M, N, K);
  if (rc) return rc;
  if ((rc = check_plan(*plan, M, N, K, true))) return rc;
  return ok();
}

size_t mxfp4_plan_workspace_bytes(const mxfp4_plan* plan, int M, int N, int K) {
  if (!plan || check_gemm_shape(M, N, K) != MXFP4_OK) return 0;
  if (check_plan(*plan, M, N, K, true) != MXFP4_OK) return 0;
  return ws_layout(*plan, M, N, K, false).total();
}

size_t mxfp4_plan_workspace_zero_bytes(const mxfp4_plan* plan, int M, int N, int K) {
  if (!plan || check_gemm_shape(M, N, K) != MXFP4_OK) return 0;
  if (check_plan(*plan, M, N, K, false) != MXFP4_OK) return 0;
  return ws_layout(*plan, M, N, K, false).zero_bytes();
}

size_t mxfp4_gemm_prequant_workspace_bytes(const mxfp4_plan* plan, int M, int N, int K) {
  if (check_gemm_shape(M, N, K) != MXFP4_OK) return 0;
  mxfp4_plan p = plan ? *plan : default_plan(M, N, K);
  if (p.mode != MXFP4_MODE_TILED && p.mode != MXFP4_MODE_STREAM) p.mode = MXFP4_MODE_PREQUANT;
  if (check_plan(p, M, N, K, false) != MXFP4_OK) return 0;
  return ws_layout(p, M, N, K, true).total();
}

size_t mxfp4_gemm_workspace_bytes(int M, int N, int K) {
  if (check_gemm_shape(M, N, K) != MXFP4_OK) return 0;
  const mxfp4_plan p = default_plan(M, N, K);
  return ws_layout(p, M, N, K, false).total();
}

}  // extern "C"

namespace {

// Argument checks of mxfp4_gemm_ex that do not depend on the plan.
int check_gemm_args(const uint16_t* a, int lda, const void* b_packed, size_t b_packed_bytes,
                    const uint16_t* c, int ldc, int M, int N, int K) {
  int rc;
  if ((rc = check_stream_ptrs(a, "a")) || (rc = check_stream_ptrs(b_packed, "b_packed")) ||
      (rc = check_stream_ptrs(c, "c")))
    return rc;
  if ((rc = check_gemm_shape(M, N, K, true))) return rc;
  if (lda < K || lda % 8 != 0) return fail(MXFP4_EINVAL, "lda must be >= K and a multiple of 8 (got %d)", lda);
  if (ldc < N) return fail(MXFP4_EINVAL, "ldc must be >= N (got %d)", ldc);
  if (!aligned(a, 16) || !aligned(b_packed, 16) || !aligned(c, 2))
    return fail(MXFP4_EINVAL, "a and b_packed must be 16-byte aligned, c 2-byte aligned");
  const size_t bneed = mxfp4_packed_bytes(N, K);
  if (b_packed_bytes < bneed)
    return fail(MXFP4_ESIZE, "b_packed holds %zu bytes, layout needs %zu", b_packed_bytes, bneed);
  return MXFP4_OK;
}

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

// This device's scratch pointer (looked up on the device's first call).
int device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MXFP4_EINVAL, "mxfp4_gemm_noalloc supports devices 0..%d (current device %d)",
                kScratchDevices - 1, dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p || !aligned(p, 256)) return fail(MXFP4_EHIP, "scratch symbol has no usable address");
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MXFP4_OK;
}

}  // namespace

extern "C" {

int mxfp4_gemm_ex(const uint16_t* a, int lda, const void* b_packed, size_t b_packed_bytes,
                  uint16_t* c, int ldc, int M, int N, int K, void* workspace,
                  size_t workspace_bytes, const mxfp4_plan* plan, void* stream) {
  if (empty_call(M, N, K)) return ok();
  int rc;
  if ((rc = check_gemm_args(a, lda, b_packed, b_packed_bytes, c, ldc, M, N, K))) return rc;
  const mxfp4_plan p = plan ? *plan : default_plan(M, N, K);
  if ((rc = check_plan(p, M, N, K, true))) return rc;
  const WsLayout wl = ws_layout(p, M, N, K, false);
  if ((rc = check_workspace(workspace, workspace_bytes, wl.total()))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const void* a_src = a;
  if (p.mode == MXFP4_MODE_PREQUANT || p.mode == MXFP4_MODE_TILED || p.mode == MXFP4_MODE_STREAM) {
    mx::launch_quant_packed(a, M, K, lda, ws + wl.a_off(), st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "quant_a_packed launch");
    a_src = ws + wl.a_off();
  }
  if (p.mode == MXFP4_MODE_TILED) {
    hipError_t e = mx::launch_gemm_tiled(static_cast<const uint8_t*>(a_src),
                                         static_cast<const uint8_t*>(b_packed), c, ldc, M, N, K,
                                         tiled_width(p), p.split_k,
                                         reinterpret_cast<float*>(ws + wl.part_off()), st);
    if (e != hipSuccess) return hip_fail(e, "gemm_tiled launch");
    return ok();
  }
  if (p.mode == MXFP4_MODE_STREAM) {
    hipError_t e = mx::launch_gemm_stream(p.m_blocks, p.n_tiles_per_wave, p.k_steps_per_wave,
                                          static_cast<const uint8_t*>(a_src),
                                          static_cast<const uint8_t*>(b_packed), c, ldc, M, N, K,
                                          reinterpret_cast<float*>(ws + wl.part_off()), st);
    if (e != hipSuccess) return hip_fail(e, "gemm_stream launch");
    return ok();
  }
  hipError_t e = mx::launch_gemm(to_internal(p), a_src, lda, static_cast<const uint8_t*>(b_packed), c,
                                 ldc, M, N, K, reinterpret_cast<float*>(ws + wl.part_off()),
                                 reinterpret_cast<unsigned*>(ws), st);
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

int mxfp4_gemm(const uint16_t* a, int lda, const void* b_packed, size_t b_packed_bytes,
               uint16_t* c, int ldc, int M, int N, int K, void* workspace,
               size_t workspace_bytes, void* stream) {
  return mxfp4_gemm_ex(a, lda, b_packed, b_packed_bytes, c, ldc, M, N, K, workspace,
                       workspace_bytes, nullptr, stream);
}

size_t mxfp4_gemm_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

int mxfp4_gemm_noalloc(const uint16_t* a, int lda, const void* b_packed, size_t b_packed_bytes,
                       uint16_t* c, int ldc, int M, int N, int K, void* stream) {
  if (empty_call(M, N, K)) return ok();
  int rc;
  if ((rc = check_gemm_args(a, lda, b_packed, b_packed_bytes, c, ldc, M, N, K))) return rc;
  const mxfp4_plan p = default_plan(M, N, K);
  if ((rc = check_plan(p, M, N, K, true))) return rc;
  const WsLayout wl = ws_layout(p, M, N, K, false);
  if (wl.total() > kNoAllocScratchBytes)
    return fail(MXFP4_EWORKSPACE,
                "the default plan for %dx%dx%d needs %zu bytes of scratch; mxfp4_gemm_noalloc "
                "holds at most %zu (call mxfp4_gemm with a workspace instead)",
                M, N, K, wl.total(), kNoAllocScratchBytes);
  void* ws = nullptr;
  if (wl.total() > 0 && (rc = device_scratch(&ws))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (wl.zero_bytes() > 0) {  // the previous call's contents stay in the array
    hipError_t e = mx::launch_zero_fill(ws, wl.zero_bytes(), st);
    if (e != hipSuccess) return hip_fail(e, "zero-fill launch");
  }
  return mxfp4_gemm_ex(a, lda, b_packed, b_packed_bytes, c, ldc, M, N, K, ws, wl.total(), &p,
                       stream);
}

int mxfp4_gemm_prequant(const void* a_packed, size_t a_packed_bytes, const void* b_packed,
                        size_t b_packed_bytes, uint16_t* c, int ldc, int M, int N, int K,
                        void* workspace, size_t workspace_bytes, const mxfp4_plan* plan,
                        void* stream) {
  if (empty_call(M, N, K)) return ok();
  int rc;
  if ((rc = check_stream_ptrs(a_packed, "a_packed")) || (rc = check_stream_ptrs(b_packed, "b_packed")) ||
      (rc = check_stream_ptrs(c, "c")))
    return rc;
  if ((rc = check_gemm_shape(M, N, K, true))) return rc;
  if (ldc < N) return fail(MXFP4_EINVAL, "ldc must be >= N (got %d)", ldc);
  if (!aligned(a_packed, 16) || !aligned(b_packed, 16) || !aligned(c, 2))
    return fail(MXFP4_EINVAL, "a_packed and b_packed must be 16-byte aligned, c 2-byte aligned");
  const size_t aneed = mxfp4_packed_bytes(M, K), bneed = mxfp4_packed_bytes(N, K);
  if (a_packed_bytes < aneed)
    return fail(MXFP4_ESIZE, "a_packed holds %zu bytes, layout needs %zu", a_packed_bytes, aneed);
  if (b_packed_bytes < bneed)
    return fail(MXFP4_ESIZE, "b_packed holds %zu bytes, layout needs %zu", b_packed_bytes, bneed);
  mxfp4_plan p = plan ? *plan : default_plan(M, N, K);
  if (p.mode != MXFP4_MODE_TILED && p.mode != MXFP4_MODE_STREAM) p.mode = MXFP4_MODE_PREQUANT;
  if ((rc = check_plan(p, M, N, K, false))) return rc;
  const WsLayout wl = ws_layout(p, M, N, K, true);
  if ((rc = check_workspace(workspace, workspace_bytes, wl.total()))) return rc;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (p.mode == MXFP4_MODE_TILED) {
    hipError_t e = mx::launch_gemm_tiled(static_cast<const uint8_t*>(a_packed),
                                         static_cast<const uint8_t*>(b_packed), c, ldc, M, N, K,
                                         tiled_width(p), p.split_k,
                                         reinterpret_cast<float*>(ws + wl.part_off()),
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "gemm_tiled launch");
    return ok();
  }
  if (p.mode == MXFP4_MODE_STREAM) {
    hipError_t e = mx::launch_gemm_stream(p.m_blocks, p.n_tiles_per_wave, p.k_steps_per_wave,
                                          static_cast<const uint8_t*>(a_packed),
                                          static_cast<const uint8_t*>(b_packed), c, ldc, M, N, K,
                                          reinterpret_cast<float*>(ws + wl.part_off()),
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "gemm_stream launch");
    return ok();
  }
  hipError_t e = mx::launch_gemm(to_internal(p), a_packed, 0, static_cast<const uint8_t*>(b_packed), c,
                                 ldc, M, N, K, reinterpret_cast<float*>(ws + wl.part_off()),
                                 reinterpret_cast<unsigned*>(ws), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return ok();
}

const char* mxfp4_last_error(void) { return g_err; }

const char* mxfp4_version(void) { return "mxfp4-gfx950 0.1.0"; }

}  // extern "C"
