// gemm_tiled.hip -- MXFP4 GEMM for large M on pre-quantized A, for gfx950.
//
// Both operands are MX-packed (16-row tiles, 128-K steps, the 16x16x128
// instruction's lane order).  A workgroup computes a 256 x 256 tile of C with
// four wavefronts (2 x 2, 128 x 128 each, one per SIMD so that each can hold
// its 256 accumulators and the staged loads in registers) using the 32x32x64
// block-scaled FP4 instruction, which does twice the work per operand byte of
// the 16x16x128 one.  K advances one 128-element step at a time through a
// two-stage LDS ring: the loads of step j + 1 go out into registers before
// the products of step j and are written to the other stage after them, so
// one barrier per step suffices and no global load is outstanding at it.
// (Loads straight to LDS would make the compiler wait for the next step's
// copy before every read of the current one.)  Each wavefront's operands are
// gathered from the packed blocks with per-lane LDS addresses:
//
//   32x32x64 lane L, K half h of the step (elements 64h .. 64h+63):
//     A row 32u + L%32  ->  16-row tile 2u + (L/16)%2, packed lane
//     (L%16) + 16*(2h + L/32), i.e. K-group 2h + L/32 of the step;
//   B column likewise; the scale byte of that (row, K-group) is byte j%4 of
//   the packed scale dword of the same tile and packed lane.
//
//   Result register i of lane L: row 8*(i/4) + 4*(L/32) + i%4, column L%32.
//
// Rows past M and columns past N read clamped (valid) tiles and are never
// stored.  Workgroup ids go to the 8 XCDs in turn; each XCD takes a
// contiguous range of tiles in row-major order, so the workgroups of one XCD
// share A rows in its L2.
#include <atomic>

#include "mx_internal.hpp"

namespace mx {

constexpr int kTileM = 256;
constexpr int kTileN = 256;
constexpr int kTiledThreads = 256;  // 4 wavefronts
// LDS bytes of one pipeline stage: A and B data (16 blocks of 1 KiB each),
// then A and B scale dwords (16 tiles x 64 lanes x 4 B each)
constexpr int kStageA = 0;
constexpr int kStageB = 16 * 1024;
constexpr int kStageAS = 32 * 1024;
constexpr int kStageBS = 36 * 1024;
constexpr int kStageBytes = 40 * 1024;
constexpr int kTiledLds = 2 * kStageBytes;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct TiledArgs {
  const uint8_t* ap;  // MX-packed A
  const uint8_t* bp;  // MX-packed B
  uint16_t* c;        // bf16 C [M][ldc]
  int M, N, ldc;
  int MT, NT, KS, KG;  // A row tiles, B row tiles, K steps, scale dwords per lane
  int tiles_m, tiles_n, per_xcd;
};

__device__ inline f32x16 mfma32_fp4(uint4 a, uint4 b, f32x16 acc, int sa, int sb) {
  i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // format 4 = e2m1 for both operands; byte 0 of each scale register
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, 4, 4, 0, sa, 0, sb);
}

__global__ __launch_bounds__(kTiledThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tiled_kernel(TiledArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // tile of this workgroup (see the file header)
  const int xcd = blockIdx.x & 7;
  const int k = blockIdx.x >> 3;
  const int tile = xcd * g.per_xcd + k;
  if (k >= g.per_xcd || tile >= g.tiles_m * g.tiles_n) return;
  const int tm = tile / g.tiles_n;
  const int tn = tile - tm * g.tiles_n;
  const int t_a0 = tm * (kTileM / 16);  // first 16-row tile of A
  const int t_b0 = tn * (kTileN / 16);  // first 16-row tile of B

  const PackedDims da = {g.MT, g.KS, g.KG};
  const PackedDims db = {g.NT, g.KS, g.KG};

  // One step's blocks pass through registers: wavefront w moves blocks w,
  // w + 4, w + 8 and w + 12 of A and of B (1 KiB each) and the scale dwords
  // of the same tiles (256 B each); tiles past the operand's last are
  // clamped.  Block addresses are wave-uniform, plus one per-lane offset.
  const size_t a_sc = da.data_bytes(), b_sc = db.data_bytes();
  // (named registers rather than arrays: arrays captured by the helpers
  // below were placed in scratch memory)
  uint4 na0, na1, na2, na3, nb0, nb1, nb2, nb3;
  uint32_t nsa0, nsa1, nsa2, nsa3, nsb0, nsb1, nsb2, nsb3;
#define MX_STAGE_LOAD(R, j)                                                                      \
  {                                                                                              \
    const int blk = wave + 4 * R;                                                                \
    const int ta = min(t_a0 + blk, g.MT - 1);                                                    \
    const int tb = min(t_b0 + blk, g.NT - 1);                                                    \
    na##R = *reinterpret_cast<const uint4*>(g.ap + ((size_t)ta * g.KS + (j)) * kBlockBytes +     \
                                            lane * 16);                                          \
    nb##R = *reinterpret_cast<const uint4*>(g.bp + ((size_t)tb * g.KS + (j)) * kBlockBytes +     \
                                            lane * 16);                                          \
    nsa##R = *reinterpret_cast<const uint32_t*>(                                                 \
        g.ap + a_sc + ((size_t)ta * g.KG + ((j) >> 2)) * 256 + lane * 4);                        \
    nsb##R = *reinterpret_cast<const uint32_t*>(                                                 \
        g.bp + b_sc + ((size_t)tb * g.KG + ((j) >> 2)) * 256 + lane * 4);                        \
  }
#define MX_STAGE_STORE(R, base)                                                                  \
  {                                                                                              \
    const int blk = wave + 4 * R;                                                                \
    *reinterpret_cast<uint4*>(base + kStageA + blk * 1024 + lane * 16) = na##R;                  \
    *reinterpret_cast<uint4*>(base + kStageB + blk * 1024 + lane * 16) = nb##R;                  \
    *reinterpret_cast<uint32_t*>(base + kStageAS + blk * 256 + lane * 4) = nsa##R;               \
    *reinterpret_cast<uint32_t*>(base + kStageBS + blk * 256 + lane * 4) = nsb##R;               \
  }
  auto load = [&](int j) {
    MX_STAGE_LOAD(0, j)
    MX_STAGE_LOAD(1, j)
    MX_STAGE_LOAD(2, j)
    MX_STAGE_LOAD(3, j)
  };
  auto store = [&](int st) {
    uint8_t* base = smem + st * kStageBytes;
    MX_STAGE_STORE(0, base)
    MX_STAGE_STORE(1, base)
    MX_STAGE_STORE(2, base)
    MX_STAGE_STORE(3, base)
  };
#undef MX_STAGE_LOAD
#undef MX_STAGE_STORE

  const int wm = wave >> 1;  // 0..1: rows 128*wm
  const int wn = wave & 1;   // 0..1: columns 128*wn
  const int half_tile = (lane >> 4) & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = f32x16{};

  load(0);
  store(0);
  for (int j = 0; j < g.KS; ++j) {
    const int st = j & 1;
    __syncthreads();  // step j is in stage st; every read of stage st ^ 1 is done
    // the last step loads its own blocks again (in bounds, never stored):
    // an unconditional load keeps the staging registers out of scratch
    load(min(j + 1, g.KS - 1));
    // keep the products of step j between the loads and the stores of step
    // j + 1, so the wait for those loads falls after the products are issued
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* base = smem + st * kStageBytes;
    const int sbyte = j & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pl = (lane & 15) + 16 * (2 * h + (lane >> 5));  // packed lane
      uint4 a[4], b[4];
      int sa[4], sb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = 8 * wm + 2 * u + half_tile;
        a[u] = *reinterpret_cast<const uint4*>(base + kStageA + t * 1024 + pl * 16);
        sa[u] = base[kStageAS + t * 256 + pl * 4 + sbyte];
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 8 * wn + 2 * v + half_tile;
        b[v] = *reinterpret_cast<const uint4*>(base + kStageB + t * 1024 + pl * 16);
        sb[v] = base[kStageBS + t * 256 + pl * 4 + sbyte];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = mfma32_fp4(a[u], b[v], acc[u][v], sa[u], sb[v]);
      __builtin_amdgcn_sched_barrier(0);  // one half's operands live at a time
    }
    // unconditional (a branch here lets the compiler move the products
    // below the stores): on the last step this rewrites the other stage,
    // which every wavefront finished reading before this step's barrier
    __builtin_amdgcn_sched_barrier(0);
    store(st ^ 1);
  }

  // epilogue: bf16, nearest even; rows >= M and columns >= N are not stored
  const int row0 = tm * kTileM + 128 * wm + 4 * (lane >> 5);
  const int col0 = tn * kTileN + 128 * wn + (lane & 31);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int col = col0 + 32 * v;
      if (col >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = row0 + 32 * u + 8 * (i >> 2) + (i & 3);
        if (row < g.M) g.c[(size_t)row * g.ldc + col] = f32_to_bf16_rne(acc[u][v][i]);
      }
    }
}

TiledGeom tiled_geometry(int M, int N, int K) {
  TiledGeom t;
  t.tiles_m = (int)(((long long)M + kTileM - 1) / kTileM);
  t.tiles_n = (int)(((long long)N + kTileN - 1) / kTileN);
  const long long tiles = (long long)t.tiles_m * t.tiles_n;
  t.per_xcd = (int)((tiles + 7) / 8);
  t.grid = 8LL * t.per_xcd;
  t.threads = kTiledThreads;
  t.lds = kTiledLds;
  (void)K;
  return t;
}

hipError_t launch_gemm_tiled(const uint8_t* a_packed, const uint8_t* b_packed, uint16_t* c, int ldc,
                             int M, int N, int K, hipStream_t stream) {
  static std::atomic<int> lds_attr_set{0};
  if (!lds_attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tiled_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kTiledLds);
    if (e != hipSuccess) return e;
    lds_attr_set.store(1, std::memory_order_release);
  }
  const TiledGeom t = tiled_geometry(M, N, K);
  const PackedDims da = packed_dims(M, K), db = packed_dims(N, K);
  TiledArgs args;
  args.ap = a_packed;
  args.bp = b_packed;
  args.c = c;
  args.M = M;
  args.N = N;
  args.ldc = ldc;
  args.MT = da.RT;
  args.NT = db.RT;
  args.KS = da.KS;
  args.KG = da.KG;
  args.tiles_m = t.tiles_m;
  args.tiles_n = t.tiles_n;
  args.per_xcd = t.per_xcd;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_tiled_kernel), dim3((unsigned)t.grid),
                         dim3(t.threads), kargs, (unsigned)t.lds, stream);
}

}  // namespace mx
