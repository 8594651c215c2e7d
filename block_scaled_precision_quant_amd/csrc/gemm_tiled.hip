// gemm_tiled.hip -- MXFP4 GEMM for large M on pre-quantized A, for gfx950.
//
// Both operands are MX-packed (16-row tiles, 128-K steps, the 16x16x128
// instruction's lane order).  A workgroup computes a 256 x 256 tile of C with
// four wavefronts (2 x 2, 128 x 128 each, one per SIMD so that each can hold
// its 256 accumulators and the staged loads in registers) using the 32x32x64
// block-scaled FP4 instruction, which does twice the work per operand byte of
// the 16x16x128 one.  K advances one 128-element step at a time through a
// two-stage LDS ring fed from two register sets: a step's global loads are
// issued two steps before its products and written to LDS after the products
// of the step before it, so one barrier per step suffices and the loads have
// two steps' worth of products to arrive.  (Loads straight to LDS would make
// the compiler wait for the next step's copy before every read of the
// current one.)  Each wavefront's operands are gathered from the packed
// blocks with per-lane LDS addresses:
//
//   32x32x64 lane L, K half h of the step (elements 64h .. 64h+63):
//     A row 32u + L%32  ->  16-row tile 2u + (L/16)%2, packed lane
//     (L%16) + 16*(2h + L/32), i.e. K-group 2h + L/32 of the step;
//   B column likewise; the scale byte of that (row, K-group) is byte j%4 of
//   the packed scale dword of the same tile and packed lane.
//
//   B is the instruction's first operand, so result register i of lane L
//   holds row L%32 and column 8*(i/4) + 4*(L/32) + i%4: four neighbouring
//   columns per register group, stored as one 8-byte write.
//
// Rows past M and columns past N read clamped (valid) tiles and are never
// stored.  Workgroup ids go to the 8 XCDs in turn; each XCD takes a
// contiguous range of tiles, ordered in groups of four tile rows walked
// column by column, so the workgroups running together on one XCD cover a
// compact block of C and share both A rows and B columns in its L2.
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
// tile order: groups of kGroupM tile rows, column-major inside a group, so
// the tiles that run at the same time on one XCD form a compact block
constexpr int kGroupM = 4;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct TiledArgs {
  const uint8_t* ap;  // MX-packed A
  const uint8_t* bp;  // MX-packed B
  uint16_t* c;        // bf16 C [M][ldc]
  int M, N, ldc;
  int MT, NT, KS, KG;  // A row tiles, B row tiles, K steps, scale dwords per lane
  int tiles_m, tiles_n, per_xcd;
};

// Raw buffer access: descriptor word 3 for untyped dword access on CDNA3/4;
// reads past num_records return zero.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;

__device__ inline BufRsrc make_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, kBufWord3);
}
__device__ inline uint4 load16(BufRsrc r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint32_t load4(BufRsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

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
  const int group = tile / (kGroupM * g.tiles_n);
  const int first_m = group * kGroupM;
  const int rows_in = min(kGroupM, g.tiles_m - first_m);
  const int in_group = tile - group * kGroupM * g.tiles_n;
  const int tm = first_m + in_group % rows_in;
  const int tn = in_group / rows_in;
  const int t_a0 = tm * (kTileM / 16);  // first 16-row tile of A
  const int t_b0 = tn * (kTileN / 16);  // first 16-row tile of B

  const PackedDims da = {g.MT, g.KS, g.KG};
  const PackedDims db = {g.NT, g.KS, g.KG};

  // One step's blocks pass through registers: wavefront w moves blocks w,
  // w + 4, w + 8 and w + 12 of A and of B (1 KiB each) and the scale dwords
  // of the same tiles (256 B each); tiles past the operand's last are
  // clamped.  Two register sets (x and y) alternate, so a step's loads are
  // issued two steps before its products.  Named registers rather than
  // arrays: arrays captured by helpers were placed in scratch memory.
  //
  // Loads go through buffer descriptors that cover just this workgroup's
  // tiles (offsets from the first tile fit in 32 bits for K <= 2^22), so an
  // address is one per-lane constant plus a wave-uniform offset.
  const int a_tiles = min(kTileM / 16, g.MT - t_a0);
  const int b_tiles = min(kTileN / 16, g.NT - t_b0);
  const size_t a_sc = da.data_bytes(), b_sc = db.data_bytes();
  const BufRsrc ra = make_rsrc(g.ap + (size_t)t_a0 * g.KS * kBlockBytes, a_tiles * g.KS * kBlockBytes);
  const BufRsrc rb = make_rsrc(g.bp + (size_t)t_b0 * g.KS * kBlockBytes, b_tiles * g.KS * kBlockBytes);
  const BufRsrc ras = make_rsrc(g.ap + a_sc + (size_t)t_a0 * g.KG * 256, a_tiles * g.KG * 256);
  const BufRsrc rbs = make_rsrc(g.bp + b_sc + (size_t)t_b0 * g.KG * 256, b_tiles * g.KG * 256);
  const int lane16 = lane * 16, lane4 = lane * 4;
  uint4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
  uint32_t xsa0, xsa1, xsa2, xsa3, xsb0, xsb1, xsb2, xsb3;
  uint4 ya0, ya1, ya2, ya3, yb0, yb1, yb2, yb3;
  uint32_t ysa0, ysa1, ysa2, ysa3, ysb0, ysb1, ysb2, ysb3;
#define MX_STAGE_LOAD(S, R, j)                                                                   \
  {                                                                                              \
    const int blk = wave + 4 * R;                                                                \
    const int ta = min(blk, a_tiles - 1);                                                        \
    const int tb = min(blk, b_tiles - 1);                                                        \
    S##a##R = load16(ra, lane16, (ta * g.KS + (j)) * kBlockBytes);                               \
    S##b##R = load16(rb, lane16, (tb * g.KS + (j)) * kBlockBytes);                               \
    S##sa##R = load4(ras, lane4, (ta * g.KG + ((j) >> 2)) * 256);                                \
    S##sb##R = load4(rbs, lane4, (tb * g.KG + ((j) >> 2)) * 256);                                \
  }
#define MX_STAGE_STORE(S, R, base)                                                               \
  {                                                                                              \
    const int blk = wave + 4 * R;                                                                \
    *reinterpret_cast<uint4*>(base + kStageA + blk * 1024 + lane * 16) = S##a##R;                \
    *reinterpret_cast<uint4*>(base + kStageB + blk * 1024 + lane * 16) = S##b##R;                \
    *reinterpret_cast<uint32_t*>(base + kStageAS + blk * 256 + lane * 4) = S##sa##R;             \
    *reinterpret_cast<uint32_t*>(base + kStageBS + blk * 256 + lane * 4) = S##sb##R;             \
  }
  auto load_x = [&](int j) {
    MX_STAGE_LOAD(x, 0, j)
    MX_STAGE_LOAD(x, 1, j)
    MX_STAGE_LOAD(x, 2, j)
    MX_STAGE_LOAD(x, 3, j)
  };
  auto load_y = [&](int j) {
    MX_STAGE_LOAD(y, 0, j)
    MX_STAGE_LOAD(y, 1, j)
    MX_STAGE_LOAD(y, 2, j)
    MX_STAGE_LOAD(y, 3, j)
  };
  auto store_x = [&](int st) {
    uint8_t* base = smem + st * kStageBytes;
    MX_STAGE_STORE(x, 0, base)
    MX_STAGE_STORE(x, 1, base)
    MX_STAGE_STORE(x, 2, base)
    MX_STAGE_STORE(x, 3, base)
  };
  auto store_y = [&](int st) {
    uint8_t* base = smem + st * kStageBytes;
    MX_STAGE_STORE(y, 0, base)
    MX_STAGE_STORE(y, 1, base)
    MX_STAGE_STORE(y, 2, base)
    MX_STAGE_STORE(y, 3, base)
  };
#undef MX_STAGE_LOAD
#undef MX_STAGE_STORE

  const int wm = wave >> 1;  // 0..1: rows 128*wm
  const int wn = wave & 1;   // 0..1: columns 128*wn
  const int half_tile = (lane >> 4) & 1;
  // acc[u][v]: rows 32u.., columns 32v.. of the wavefront's 128 x 128; B is
  // the instruction's first operand, so lane L holds row L%32 and columns
  // 8*(i/4) + 4*(L/32) + i%4 (four neighbours per register group)
  f32x16 acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = f32x16{};

  // Operands of one half of a K step (64 elements) for the wavefront's
  // 4 x 4 products: P holds K half 0, Q K half 1.  Per-lane LDS offsets of
  // half 0; half 1 is 512 bytes further for codes and 128 for scales, tile
  // u (or v) 2048 and 512 further, stage 1 kStageBytes further.
  const int pl0 = (lane & 15) + 16 * (lane >> 5);  // packed lane, K half 0
  const int off_a = kStageA + (8 * wm + half_tile) * 1024 + pl0 * 16;
  const int off_b = kStageB + (8 * wn + half_tile) * 1024 + pl0 * 16;
  const int off_as = kStageAS + (8 * wm + half_tile) * 256 + pl0 * 4;
  const int off_bs = kStageBS + (8 * wn + half_tile) * 256 + pl0 * 4;
  uint4 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3;
  int psa0, psa1, psa2, psa3, psb0, psb1, psb2, psb3;
  int qsa0, qsa1, qsa2, qsa3, qsb0, qsb1, qsb2, qsb3;
#define MX_LDS16(off) (*reinterpret_cast<const uint4*>(smem + (off)))
  // S = p or q, half h, stage st, scale byte sbyte (K step % 4)
#define MX_READ(S, st, h, sbyte)                                                                 \
  {                                                                                              \
    const int o = (st) * kStageBytes + (h) * 512;                                                \
    const int os = (st) * kStageBytes + (h) * 128 + (sbyte);                                     \
    S##a0 = MX_LDS16(off_a + o);                                                                 \
    S##a1 = MX_LDS16(off_a + o + 2048);                                                          \
    S##a2 = MX_LDS16(off_a + o + 4096);                                                          \
    S##a3 = MX_LDS16(off_a + o + 6144);                                                          \
    S##b0 = MX_LDS16(off_b + o);                                                                 \
    S##b1 = MX_LDS16(off_b + o + 2048);                                                          \
    S##b2 = MX_LDS16(off_b + o + 4096);                                                          \
    S##b3 = MX_LDS16(off_b + o + 6144);                                                          \
    S##sa0 = smem[off_as + os];                                                                  \
    S##sa1 = smem[off_as + os + 512];                                                            \
    S##sa2 = smem[off_as + os + 1024];                                                           \
    S##sa3 = smem[off_as + os + 1536];                                                           \
    S##sb0 = smem[off_bs + os];                                                                  \
    S##sb1 = smem[off_bs + os + 512];                                                            \
    S##sb2 = smem[off_bs + os + 1024];                                                           \
    S##sb3 = smem[off_bs + os + 1536];                                                           \
  }
#define MX_ROW(S, u)                                                                             \
  acc[u][0] = mfma32_fp4(S##b0, S##a##u, acc[u][0], S##sb0, S##sa##u);                            \
  acc[u][1] = mfma32_fp4(S##b1, S##a##u, acc[u][1], S##sb1, S##sa##u);                            \
  acc[u][2] = mfma32_fp4(S##b2, S##a##u, acc[u][2], S##sb2, S##sa##u);                            \
  acc[u][3] = mfma32_fp4(S##b3, S##a##u, acc[u][3], S##sb3, S##sa##u);
#define MX_MFMA(S) \
  { MX_ROW(S, 0) MX_ROW(S, 1) MX_ROW(S, 2) MX_ROW(S, 3) }
  // one step in stage st (K step j): the loads of step j + 2 into register
  // set L interleaved with the products of half 0, the blocks of step j + 1
  // from register set W written to the other stage, the barrier, the half-0
  // operands of step j + 1 read, the products of half 1, the half-1 operands
  // of step j + 1 read
#define MX_STEP(st, j, L, W)                                                                     \
  {                                                                                              \
    load_##L(min((j) + 2, last));                                                                \
    MX_MFMA(p)                                                                                   \
    store_##W(1 - (st));                                                                         \
    for (int i = 0; i < 12; ++i) {                                                               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */                              \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* global load */                       \
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0); /* LDS write */                         \
    }                                                                                            \
    for (int i = 0; i < 4; ++i) {                                                                \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                         \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                         \
    }                                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    __syncthreads();                                                                             \
    MX_READ(p, 1 - (st), 0, ((j) + 1) & 3)                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MX_MFMA(q)                                                                                   \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MX_READ(q, 1 - (st), 1, ((j) + 1) & 3)                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                           \
  }

  // Step j uses stage j % 2 and runs as one MX_STEP: at its start, its
  // operands are being read and register set W holds the blocks of step
  // j + 1 (loaded during step j - 1).  The barrier sits between the two
  // halves' products; at it every wavefront has finished reading stage
  // j % 2's operands for step j (the barrier waits for all LDS accesses)
  // and has written step j + 1's blocks, so the step after next may
  // overwrite stage j % 2 and step j + 1's operands may be read, while the
  // products of half 1 keep the matrix cores busy across it.  Steps past
  // the last load and read the last step again (in bounds, never used):
  // unconditional loads keep the register sets out of scratch.  The loop
  // takes whole pairs of steps; an odd last step follows it.
  const int last = g.KS - 1;
  load_x(0);
  load_y(min(1, last));
  store_x(0);
  __syncthreads();
  MX_READ(p, 0, 0, 0)
  MX_READ(q, 0, 1, 0)
  int j = 0;
  for (; j + 1 < g.KS; j += 2) {
    MX_STEP(0, j, x, y)
    MX_STEP(1, j + 1, y, x)
  }
  if (j < g.KS) {  // odd KS: the last step is in stage 0, its operands read
    MX_MFMA(p)
    MX_MFMA(q)
  }
#undef MX_STEP
#undef MX_MFMA
#undef MX_ROW
#undef MX_READ
#undef MX_LDS16

  // epilogue: bf16, nearest even; rows >= M and columns >= N are not
  // stored.  Four neighbouring columns go out as one 8-byte store when the
  // whole tile lies inside N and C's rows are 8-byte aligned; otherwise one
  // element at a time.
  const int row0 = tm * kTileM + 128 * wm + (lane & 31);
  const int col0 = tn * kTileN + 128 * wn + 4 * (lane >> 5);
  const bool vec = (g.ldc % 4 == 0) && ((reinterpret_cast<uintptr_t>(g.c) & 7) == 0) &&
                   (tn + 1) * kTileN <= g.N;
  if (vec) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = row0 + 32 * u;
      if (row >= g.M) continue;
      uint16_t* crow = g.c + (size_t)row * g.ldc + col0;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo = f32_to_bf16_rne(acc[u][v][4 * q]) |
                              ((uint32_t)f32_to_bf16_rne(acc[u][v][4 * q + 1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc[u][v][4 * q + 2]) |
                              ((uint32_t)f32_to_bf16_rne(acc[u][v][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(crow + 32 * v + 8 * q) = make_uint2(lo, hi);
        }
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = row0 + 32 * u;
      if (row >= g.M) continue;
      uint16_t* crow = g.c + (size_t)row * g.ldc;
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int col = col0 + 32 * v + 8 * (i >> 2) + (i & 3);
          if (col < g.N) crow[col] = f32_to_bf16_rne(acc[u][v][i]);
        }
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
