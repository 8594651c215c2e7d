// mx_internal.hpp -- declarations shared between the kernel files and the
// C-ABI layer (api.cpp).  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_device.hpp"

namespace mx {

// Tiling of one GEMM call (mirrors the public mxfp4_plan).
struct Plan {
  int mode;      // 1 fused, 2 prequant
  int mbw;       // 16-row A blocks per workgroup
  int ntw;       // 16-column B tiles per wavefront
  int wn;        // wavefronts along N
  int wk;        // wavefronts along K
  int ksw;       // 128-K steps per wavefront
  int split;     // workgroups along K
  int reduce;    // split > 1: how the K slices are summed (Reduce)
};

// Split-K reductions (values match MXFP4_REDUCE_* in mxfp4.h).
enum Reduce : int {
  kReduceKernel = 0,  // fp32 partials [split][M][N], splitk_reduce_kernel
  kReduceLastWg = 1,  // fp32 partials; the last workgroup of each tile sums them
  kReduceAtomic = 2,  // fp32 atomic adds into one [M][N] accumulator; the last
                      // workgroup of each tile converts it and clears it
};

constexpr int kMaxLds = 160 * 1024;
constexpr int kAPT = 8;              // fused A chunks per wavefront per load round (16 B per lane each)
constexpr int kMaxLastWgSplit = 16;  // split_k bound for the last-workgroup reduce
constexpr int kMaxThreads = 512;

// Launch geometry derived from a plan and a shape.
struct GemmGeom {
  int MT, NT, KS, KG;
  int mgroups, ngroups;
  int kswg;        // steps per workgroup = wk * ksw
  int ngw_max;     // scale dwords per (block, lane) the workgroup may span
  size_t lds_a;    // bytes of A data in LDS
  size_t lds_asc;  // bytes of A scales in LDS
  size_t lds_red;  // bytes of the in-block reduce area
  size_t lds_total;
  unsigned grid;
  int threads;
};

GemmGeom gemm_geometry(const Plan& p, int M, int N, int K);

// True when a kernel for (mode, mbw, ntw, ksw) is compiled in.
bool gemm_kernel_available(int mode, int mbw, int ntw, int ksw);

// Enqueue the GEMM kernel (and the split-K reduce kernel when p.split > 1
// and p.reduce == kReduceKernel).
//   a: bf16 A (fused) or MX-packed A (prequant); ws: fp32 partials
//   [split][M][N], or the zeroed [M][N] accumulator for kReduceAtomic;
//   counters: mgroups*ngroups zeroed tile counters (kReduceLastWg and
//   kReduceAtomic).
hipError_t launch_gemm(const Plan& p, const void* a, int lda, const uint8_t* b_packed,
                       uint16_t* c, int ldc, int M, int N, int K, float* ws,
                       unsigned* counters, hipStream_t stream);

// Large-M kernel on pre-quantized A (gemm_tiled.hip): 256 x tile_n tiles of
// C (tile_n 256 or 128), 32x32x64 products, K pipelined through LDS.
// Longest K of the tiled kernel: its buffer offsets within one workgroup's
// 16 row tiles stay below 2^31.
constexpr int kTiledMaxK = 1 << 22;
// split > 1 shares each tile's K among split workgroups of sps steps (a
// multiple of 4), whose fp32 partials [split][M][N] in ws the reduce kernel
// sums.
struct TiledGeom {
  int tiles_m, tiles_n, per_xcd;
  long long grid;  // workgroups
  int threads;
  int lds;         // bytes of LDS per workgroup
  int sps;         // K steps per workgroup
};
TiledGeom tiled_geometry(int M, int N, int K, int tile_n, int split);
hipError_t launch_gemm_tiled(const uint8_t* a_packed, const uint8_t* b_packed, uint16_t* c, int ldc,
                             int M, int N, int K, int tile_n, int split, float* ws,
                             hipStream_t stream);

// Sum fp32 partials [S][M][N] in order s = 0..S-1 into bf16 C (gemm.hip).
hipError_t launch_splitk_reduce(const float* ws, uint16_t* c, int M, int N, int ldc, int S,
                                hipStream_t stream);

// K-looping kernel on pre-quantized A (gemm_stream.hip): four wavefronts
// along N, MBW row blocks, NTW tiles per wavefront, steps_per_wg 128-K steps
// per workgroup (a multiple of 4), K split over ceil(ceil(KS/4) / chunks)
// workgroups whose fp32 partials the reduce kernel sums.
constexpr int kStreamMaxK = 1 << 22;  // buffer offsets within a workgroup's tiles stay below 2^31
struct StreamGeom {
  int MT, NT, KS, KG;
  int chunks, split;   // 4-step chunks per workgroup, workgroups along K
  int mgroups, ngroups;
  long long grid;      // workgroups
  int threads;
  int lds;             // bytes of LDS per workgroup (static)
};
bool stream_kernel_available(int mbw, int ntw);
StreamGeom stream_geometry(int mbw, int ntw, int steps_per_wg, int M, int N, int K);
hipError_t launch_gemm_stream(int mbw, int ntw, int steps_per_wg, const uint8_t* a_packed,
                              const uint8_t* b_packed, uint16_t* c, int ldc, int M, int N, int K,
                              float* ws, hipStream_t stream);

// Zero `bytes` bytes (a multiple of 4) at p with a fill kernel.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

void launch_quant_linear(const uint16_t* a, int M, int K, int lda, uint8_t* out_fp4, int ld_fp4,
                         uint8_t* out_scale, int ld_scale, hipStream_t stream);
void launch_quant_packed(const uint16_t* a, int M, int K, int lda, uint8_t* out,
                         hipStream_t stream);
void launch_pack_b(const uint8_t* b_fp4, const uint8_t* b_scale, int N, int K, uint8_t* out,
                   hipStream_t stream);

}  // namespace mx
