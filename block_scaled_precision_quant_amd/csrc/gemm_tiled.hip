// gemm_tiled.hip -- MXFP4 GEMM for large M on pre-quantized A, for gfx950.
//
// Both operands are MX-packed (16-row tiles, 128-K steps, the 16x16x128
// instruction's lane order).  A workgroup computes a 256 x 256 tile of C with
// eight wavefronts (2 x 4, 128 x 64 each), or a 256 x 128 tile with eight
// wavefronts of 64 x 64 (4 x 2) -- two per SIMD: each holds its
// accumulators and two halves' operands in registers, and one wavefront's
// waits are covered by the other's products -- using the 32x32x64
// block-scaled FP4 instruction, which does twice the work per
// operand byte of the 16x16x128 one.  K advances one 128-element step at a
// time through a four-stage LDS ring (40 KiB per stage, all 160 KiB of the
// CU) filled by direct global-to-LDS copies, issued three steps ahead of
// their use with no register staging.  One barrier per step, placed between
// the products of the step's two K halves, so the matrix cores stay busy
// across it.  Each wavefront's operands are gathered from the packed blocks
// with per-lane LDS addresses:
//
//   32x32x64 lane L, K half h of the step (elements 64h .. 64h+63):
//     A row 32u + L%32  ->  16-row tile 2u + (L/16)%2, packed lane
//     (L%16) + 16*(2h + L/32), i.e. K-group 2h + L/32 of the step;
//   B column likewise; the scale byte of that (row, K-group) is byte j%4 of
//   the packed scale dword of the same tile and packed lane, which the
//   instruction selects itself.
//
//   B is the instruction's first operand, so result register i of lane L
//   holds row L%32 and column 8*(i/4) + 4*(L/32) + i%4: four neighbouring
//   columns per register group.  The epilogue rounds them to bf16, stages
//   each wavefront's block in LDS and writes it back as whole rows.
//
// Rows past M and columns past N read clamped (valid) tiles and are never
// stored.  Workgroup ids go to the 8 XCDs in turn; each XCD takes a
// contiguous range of tiles, ordered in groups of four tile rows walked
// column by column, so the workgroups running together on one XCD cover a
// compact block of C and share both A rows and B columns in its L2.
//
// With split > 1 (shapes with too few tiles to fill the CUs) each tile's K
// steps are shared among `split` workgroups, sps steps each (a multiple of
// four, so every range starts a scale group), and each writes its fp32
// tile into the partials [split][M][N] that the reduce kernel of gemm.hip
// sums in order.
#include "mx_internal.hpp"

namespace mx {

constexpr int kTileM = 256;
// Tiles are 256 rows x kTN columns (kTN 256 or 128); a wavefront computes
// 32 kU rows x 64 columns (kU 4 or 2), eight wavefronts per workgroup.
// LDS bytes of one pipeline stage: A and B data (16 blocks of 1 KiB each),
// then A and B scale dwords (16 tiles x 64 lanes x 4 B each)
constexpr int kStageA = 0;
constexpr int kStageB = 16 * 1024;
constexpr int kStageAS = 32 * 1024;
constexpr int kStageBS = 36 * 1024;
constexpr int kStageBytes = 40 * 1024;
// tile order: groups of kGroupM tile rows, column-major inside a group, so
// the tiles that run at the same time on one XCD form a compact block
constexpr int kGroupM = 4;

// The four pipeline stages (160 KiB, all of a CU's LDS), as separate
// arrays: the compiler then tracks the asynchronous copies into each stage
// on their own, so a read of one stage waits only for the copies into it.
__shared__ __align__(16) uint8_t g_stage0[kStageBytes];
__shared__ __align__(16) uint8_t g_stage1[kStageBytes];
__shared__ __align__(16) uint8_t g_stage2[kStageBytes];
__shared__ __align__(16) uint8_t g_stage3[kStageBytes];

// Copies with the nontemporal hint, for an operand that so few workgroups
// read that it streams from HBM.  B's, for grids of at most four row tiles:
// 8-18 % less time per call at 1024x8192x8192, 768x8192x8192,
// 256x4096x14336 and the split 256/512 x 8192 x 28672 plans, 2-4 % at
// 1024x16384x16384 and 384x16384x16384; with 16 and 32 row tiles (4096^3,
// 8192^3), whose B columns many tiles re-read from the L2, it cost 2-3 %.
// A's, for grids of at most eight column tiles: 4-7 % at 8192x1024x8192,
// 16384x512x4096 and 4096x1024x16384; with 64 it cost 13 %.
__device__ inline void dma16_nt(BufRsrc r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 16, voff, soff, 0, kCachePolicyNT);
}
constexpr int kNtMaxRowTiles = 4;
constexpr int kNtMaxColTiles = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

struct TiledArgs {
  const uint8_t* ap;  // MX-packed A
  const uint8_t* bp;  // MX-packed B
  uint16_t* c;        // bf16 C [M][ldc]
  float* ws;          // fp32 partials [split][M][N] (split > 1)
  int M, N, ldc;
  int MT, NT, KS, KG;  // A row tiles, B row tiles, K steps, scale dwords per lane
  int tiles_m, tiles_n, per_xcd;
  int split, sps;      // workgroups per tile along K, K steps of each (a multiple of 4)
};


// kSel selects the scale byte of sa and sb (the K step's position in its
// group of four steps)
template <int kSel>
__device__ inline f32x16 mfma32_fp4(uint4 a, uint4 b, f32x16 acc, int sa, int sb) {
  i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // format 4 = e2m1 for both operands
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc, 4, 4, kSel, sa, kSel, sb);
}

// Each wavefront waits for its own copies except the newest N instructions,
// and for its LDS accesses, then the workgroup barrier.  An asm statement:
// the compiler's barrier would wait for every copy in flight.
template <int N>
__device__ inline void wait_copies_barrier() {
  static_assert(N == 6 || N == 8 || N == 9 || N == 12 || N == 18, "copy counts of the tilings");
  if constexpr (N == 6)
    asm volatile("s_waitcnt vmcnt(6)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 9)
    asm volatile("s_waitcnt vmcnt(9)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 8)
    asm volatile("s_waitcnt vmcnt(8)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 12)
    asm volatile("s_waitcnt vmcnt(12)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(18)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int kTN, int kU, bool kNtA, bool kNtB>
__global__ __launch_bounds__(kTN * 8 / kU) __attribute__((amdgpu_waves_per_eu(kTN / (32 * kU), kTN / (32 * kU))))
void gemm_tiled_kernel(TiledArgs g) {
  constexpr int kWavesN = kTN / 64;       // wavefronts along N (64 columns each)
  constexpr int kWaves = kWavesN * 8 / kU;  // and 8 / kU along M (32 kU rows each)
  constexpr int kRA = 16 / kWaves;        // A blocks each wavefront copies per step
  constexpr int kRB = kTN / 16 / kWaves;  // B blocks each wavefront copies per step
  constexpr int kC = kRA + kRB;           // copy instructions per step (and per scale group)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // tile and K range of this workgroup (see the file header)
  const int xcd = blockIdx.x & 7;
  const int k = blockIdx.x >> 3;
  const int tiles = g.tiles_m * g.tiles_n;
  const int task = xcd * g.per_xcd + k;
  if (k >= g.per_xcd || task >= tiles * g.split) return;
  const int s = task / tiles;
  const int tile = task - s * tiles;
  const int j0 = s * g.sps;                   // first K step
  const int nsteps = min(g.sps, g.KS - j0);   // >= 1 (checked by the host)
  const int group = tile / (kGroupM * g.tiles_n);
  const int first_m = group * kGroupM;
  const int rows_in = min(kGroupM, g.tiles_m - first_m);
  const int in_group = tile - group * kGroupM * g.tiles_n;
  const int tm = first_m + in_group % rows_in;
  const int tn = in_group / rows_in;
  const int t_a0 = tm * (kTileM / 16);  // first 16-row tile of A
  const int t_b0 = tn * (kTN / 16);  // first 16-row tile of B

  const PackedDims da = {g.MT, g.KS, g.KG};
  const PackedDims db = {g.NT, g.KS, g.KG};

  // Copies: wavefront w moves blocks w and w + 8 of A and of B (1 KiB each)
  // and the scale dwords of the same tiles (256 B each) of a
  // step into that step's stage; tiles past the operand's last are clamped.
  // They go through buffer descriptors that cover just this workgroup's
  // tiles (offsets from the first tile fit in 32 bits for K <= 2^22), so an
  // address is one per-lane constant plus a wave-uniform offset.
  const int a_tiles = min(kTileM / 16, g.MT - t_a0);
  const int b_tiles = min(kTN / 16, g.NT - t_b0);
  const size_t a_sc = da.data_bytes(), b_sc = db.data_bytes();
  const BufRsrc ra = make_rsrc(g.ap + (size_t)t_a0 * g.KS * kBlockBytes, a_tiles * g.KS * kBlockBytes);
  const BufRsrc rb = make_rsrc(g.bp + (size_t)t_b0 * g.KS * kBlockBytes, b_tiles * g.KS * kBlockBytes);
  const BufRsrc ras = make_rsrc(g.ap + a_sc + (size_t)t_a0 * g.KG * 256, a_tiles * g.KG * 256);
  const BufRsrc rbs = make_rsrc(g.bp + b_sc + (size_t)t_b0 * g.KG * 256, b_tiles * g.KG * 256);
  const int lane16 = lane * 16, lane4 = lane * 4;
  int sa_[kRA], ssa_[kRA], sb_[kRB], ssb_[kRB];  // wave-uniform offsets of the wavefront's tiles
#pragma unroll
  for (int r = 0; r < kRA; ++r) {
    const int ta = min(wave + kWaves * r, a_tiles - 1);
    sa_[r] = ta * g.KS * kBlockBytes;
    ssa_[r] = ta * g.KG * 256;
  }
#pragma unroll
  for (int r = 0; r < kRB; ++r) {
    const int tb = min(wave + kWaves * r, b_tiles - 1);
    sb_[r] = tb * g.KS * kBlockBytes;
    ssb_[r] = tb * g.KG * 256;
  }
  const int last = nsteps - 1;
  // copy step j0 + jj (jj clamped to the last) into stage ST: 4
  // instructions, 8 when SC (jj % 4 == 0) adds the scale dwords of its
  // group of four steps
#define MX_DMA(ST, jj, SC)                                                                       \
  {                                                                                              \
    const int js = j0 + min((jj), last);                                                         \
    const int od = js * kBlockBytes, os = (js >> 2) * 256;                                       \
    _Pragma("unroll") for (int r = 0; r < kRA; ++r) {                                            \
      if constexpr (kNtA) dma16_nt(ra, ST + kStageA + (wave + kWaves * r) * 1024, lane16, sa_[r] + od); \
      else dma16(ra, ST + kStageA + (wave + kWaves * r) * 1024, lane16, sa_[r] + od);            \
      if (SC) dma4(ras, ST + kStageAS + (wave + kWaves * r) * 256, lane4, ssa_[r] + os);         \
    }                                                                                            \
    _Pragma("unroll") for (int r = 0; r < kRB; ++r) {                                            \
      if constexpr (kNtB) dma16_nt(rb, ST + kStageB + (wave + kWaves * r) * 1024, lane16, sb_[r] + od); \
      else dma16(rb, ST + kStageB + (wave + kWaves * r) * 1024, lane16, sb_[r] + od);            \
      if (SC) dma4(rbs, ST + kStageBS + (wave + kWaves * r) * 256, lane4, ssb_[r] + os);         \
    }                                                                                            \
  }

  const int wm = wave / kWavesN;  // rows 32*kU*wm
  const int wn = wave % kWavesN;  // columns 64*wn
  const int half_tile = (lane >> 4) & 1;
  // acc[u][v]: rows 32u.., columns 32v.. of the wavefront's block; B is
  // the instruction's first operand, so lane L holds row L%32 and columns
  // 8*(i/4) + 4*(L/32) + i%4 (four neighbours per register group)
  f32x16 acc[kU][2];
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = f32x16{};

  // Operands of one half of a K step (64 elements) for the wavefront's
  // kU x 2 products: P holds K half 0, Q K half 1.  Per-lane LDS offsets of
  // half 0; half 1 is 512 bytes further for codes and 128 for scales, tile
  // u (or v) 2048 and 512 further.  A scale dword holds the bytes of four
  // steps: it is copied with the group's first step (always into stage 0)
  // and read once, before that step; the instruction picks each step's byte.
  const int pl0 = (lane & 15) + 16 * (lane >> 5);  // packed lane, K half 0
  const int off_a = kStageA + (2 * kU * wm + half_tile) * 1024 + pl0 * 16;
  const int off_b = kStageB + (4 * wn + half_tile) * 1024 + pl0 * 16;
  const int off_as = kStageAS + (2 * kU * wm + half_tile) * 256 + pl0 * 4;
  const int off_bs = kStageBS + (4 * wn + half_tile) * 256 + pl0 * 4;
  uint4 pa0, pa1, pa2, pa3, pb0, pb1, pb2, pb3, qa0, qa1, qa2, qa3, qb0, qb1, qb2, qb3;
  int psa0, psa1, psa2, psa3, psb0, psb1, psb2, psb3;
  int qsa0, qsa1, qsa2, qsa3, qsb0, qsb1, qsb2, qsb3;
#define MX_LDS16(ST, off) (*reinterpret_cast<const uint4*>(ST + (off)))
#define MX_LDS4(ST, off) (*reinterpret_cast<const int*>(ST + (off)))
  // S = p or q, half h, stage ST; SC: the scale dwords too
#define MX_READ(S, ST, h, SC)                                                                    \
  {                                                                                              \
    S##a0 = MX_LDS16(ST, off_a + (h) * 512);                                                     \
    S##a1 = MX_LDS16(ST, off_a + (h) * 512 + 2048);                                              \
    if constexpr (kU == 4) {                                                                     \
      S##a2 = MX_LDS16(ST, off_a + (h) * 512 + 4096);                                            \
      S##a3 = MX_LDS16(ST, off_a + (h) * 512 + 6144);                                            \
    }                                                                                            \
    S##b0 = MX_LDS16(ST, off_b + (h) * 512);                                                     \
    S##b1 = MX_LDS16(ST, off_b + (h) * 512 + 2048);                                              \
    if (SC) {                                                                                    \
      S##sa0 = MX_LDS4(ST, off_as + (h) * 128);                                                  \
      S##sa1 = MX_LDS4(ST, off_as + (h) * 128 + 512);                                            \
      if constexpr (kU == 4) {                                                                   \
        S##sa2 = MX_LDS4(ST, off_as + (h) * 128 + 1024);                                         \
        S##sa3 = MX_LDS4(ST, off_as + (h) * 128 + 1536);                                         \
      }                                                                                          \
      S##sb0 = MX_LDS4(ST, off_bs + (h) * 128);                                                  \
      S##sb1 = MX_LDS4(ST, off_bs + (h) * 128 + 512);                                            \
    }                                                                                            \
  }
#define MX_ROW(S, u, k)                                                                          \
  acc[u][0] = mfma32_fp4<k>(S##b0, S##a##u, acc[u][0], S##sb0, S##sa##u);                        \
  acc[u][1] = mfma32_fp4<k>(S##b1, S##a##u, acc[u][1], S##sb1, S##sa##u);
#define MX_MFMA(S, k)                                                                            \
  {                                                                                              \
    MX_ROW(S, 0, k) MX_ROW(S, 1, k)                                                              \
    if constexpr (kU == 4) { MX_ROW(S, 2, k) MX_ROW(S, 3, k) }                                   \
  }
  // Before the barrier that precedes step j + 1's reads: own copies of
  // step j + 1 done (those of steps j + 2 and j + 3 may be in flight: N
  // instructions, 2 kC or 3 kC by where the groups' scale copies fall), own
  // LDS accesses done.
#define MX_BARRIER(N)                                                                            \
  __builtin_amdgcn_sched_barrier(0);                                                             \
  wait_copies_barrier<N>();                                                                      \
  __builtin_amdgcn_sched_barrier(0);
  // K step jj = 4i + k, in stage STC; STN is the stage of step jj + 1:
  // products of half 0; barrier; the half-0 operands of step jj + 1 read,
  // the copy of step jj + 4 into STC issued and the products of half 1, all
  // interleaved; the half-1 operands of step jj + 1 read
#define MX_STEP(k, jj, STC, STN, N)                                                              \
  {                                                                                              \
    MX_MFMA(p, k)                                                                                \
    MX_BARRIER(N)                                                                                \
    MX_READ(p, STN, 0, (k) == 3)                                                                 \
    MX_DMA(STC, (jj) + 4, (k) == 0)                                                              \
    MX_MFMA(q, k)                                                                                \
    for (int i = 0; i < 2 * kU; ++i) {                                                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); /* MFMA */                              \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); /* LDS read */                          \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); /* copy to LDS */                       \
    }                                                                                            \
    __builtin_amdgcn_sched_barrier(0);                                                           \
    MX_READ(q, STN, 1, (k) == 3)                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                           \
  }

  // Step j uses stage j % 4.  Its copy was issued three steps earlier,
  // right after the barrier at which every wavefront had finished reading
  // that stage for step j - 4; the barrier before step j's operands are
  // read follows each wavefront's wait for its own copies of step j.  The
  // barrier sits between the two halves' products, so the products of half
  // 1 keep the matrix cores busy while step j + 1's operands are read and
  // step j + 4's copy is issued.  Steps past the last copy the last step
  // again (in bounds, never used).  The loop takes groups of four steps
  // (stages and scale bytes are compile-time in each), a tail of up to three
  // follows.
  MX_DMA(g_stage0, 0, true)
  MX_DMA(g_stage1, 1, false)
  MX_DMA(g_stage2, 2, false)
  MX_DMA(g_stage3, 3, false)
  __builtin_amdgcn_sched_barrier(0);
  wait_copies_barrier<3 * kC>();  // step 0 copied (steps 1-3 may be in flight)
  __builtin_amdgcn_sched_barrier(0);
  MX_READ(p, g_stage0, 0, true)
  MX_READ(q, g_stage0, 1, true)
  int j = 0;
  for (; j + 3 < nsteps; j += 4) {
    MX_STEP(0, j, g_stage0, g_stage1, 2 * kC)
    MX_STEP(1, j + 1, g_stage1, g_stage2, 3 * kC)
    MX_STEP(2, j + 2, g_stage2, g_stage3, 3 * kC)
    MX_STEP(3, j + 3, g_stage3, g_stage0, 2 * kC)
  }
  if (j < nsteps) MX_STEP(0, j, g_stage0, g_stage1, 2 * kC)
  if (j + 1 < nsteps) MX_STEP(1, j + 1, g_stage1, g_stage2, 3 * kC)
  if (j + 2 < nsteps) MX_STEP(2, j + 2, g_stage2, g_stage3, 3 * kC)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy outlives the loop
#undef MX_STEP
#undef MX_BARRIER
#undef MX_MFMA
#undef MX_ROW
#undef MX_READ
#undef MX_LDS4
#undef MX_LDS16
#undef MX_DMA

  // epilogue: bf16, nearest even; rows >= M and columns >= N are not
  // stored.  When the whole tile lies inside N and C's rows are 16-byte
  // aligned, each wavefront stages its 32 kU x 64 block in its own half of an
  // LDS stage array (rows 144 bytes apart) and writes it back as whole rows,
  // 16 bytes per lane, nontemporal (C is not read again: at 8192^3 the call
  // takes about 3 % less time after the cache eviction than with plain
  // stores); otherwise each value goes out on its own.
  const int row0 = tm * kTileM + 32 * kU * wm;
  const int col0 = tn * kTN + 64 * wn;
  if (g.split > 1) {
    // fp32 partial of this K range: lane L holds row L%32 of each 32-row
    // block and four neighbouring columns per register group, one 16-byte
    // store each where N allows
    float* part = g.ws + (size_t)s * g.M * g.N;
    const int lrow0 = row0 + (lane & 31);
    const int lcol0 = col0 + 4 * (lane >> 5);
    const bool vec4 = (g.N % 4) == 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int row = lrow0 + 32 * u;
      if (row >= g.M) continue;
      float* prow = part + (size_t)row * g.N;
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = lcol0 + 32 * v + 8 * q;
          if (vec4 && col + 3 < g.N) {
            *reinterpret_cast<f32x4*>(prow + col) =
                f32x4{acc[u][v][4 * q], acc[u][v][4 * q + 1], acc[u][v][4 * q + 2], acc[u][v][4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < g.N) prow[col + e] = acc[u][v][4 * q + e];
          }
        }
    }
    return;
  }
  const bool vec = (g.ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(g.c) & 15) == 0) &&
                   (tn + 1) * kTN <= g.N;
  if (vec) {
    constexpr int kPitch = 144;  // bytes per staged row
    const int wp = wave >> 1;
    uint8_t* stage = (wp == 0 ? g_stage0 : wp == 1 ? g_stage1 : wp == 2 ? g_stage2 : g_stage3) + (wave & 1) * 32 * kU * kPitch;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every stage read done
    __builtin_amdgcn_sched_barrier(0);
    const int wrow = (lane & 31) * kPitch + 8 * (lane >> 5);
    const int rsub = lane >> 3, cchunk = lane & 7;
    // With 128 x 64 blocks (kU == 4) one 32-row block at a time: its rows
    // staged, then read back and stored while the next block is staged, so
    // the LDS writes overlap the stores (1-5 % less time per 256 x 256-tile
    // kernel at 2048x4096x4096 to 8192^3, the same bits); 64 x 64 blocks
    // stage all their rows first (no gain measured there).
    constexpr int kBlk = kU == 4 ? 1 : kU;
#pragma unroll
    for (int u0 = 0; u0 < kU; u0 += kBlk) {
#pragma unroll
      for (int u = u0; u < u0 + kBlk; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x2 lo = {acc[u][v][4 * q], acc[u][v][4 * q + 1]};
            const f32x2 hi = {acc[u][v][4 * q + 2], acc[u][v][4 * q + 3]};
            const uint2 w = make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                       __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2)));
            *reinterpret_cast<uint2*>(stage + wrow + 32 * u * kPitch + 2 * (32 * v + 8 * q)) = w;
          }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // these rows staged, lanes exchanged
#pragma unroll
      for (int i = 4 * u0; i < 4 * (u0 + kBlk); ++i) {
        const int r = 8 * i + rsub;
        const uint4 d = *reinterpret_cast<const uint4*>(stage + r * kPitch + 16 * cchunk);
        if (row0 + r < g.M)
          __builtin_nontemporal_store(u32x4{d.x, d.y, d.z, d.w},
                                      reinterpret_cast<u32x4*>(g.c + (size_t)(row0 + r) * g.ldc + col0 + 8 * cchunk));
      }
    }
  } else {
    const int lrow0 = row0 + (lane & 31);
    const int lcol0 = col0 + 4 * (lane >> 5);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int row = lrow0 + 32 * u;
      if (row >= g.M) continue;
      uint16_t* crow = g.c + (size_t)row * g.ldc;
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int col = lcol0 + 32 * v + 8 * (i >> 2) + (i & 3);
          if (col < g.N) crow[col] = f32_to_bf16_rne(acc[u][v][i]);
        }
    }
  }
}

TiledGeom tiled_geometry(int M, int N, int K, int tile_n, int split) {
  TiledGeom t;
  t.tiles_m = (int)(((long long)M + kTileM - 1) / kTileM);
  t.tiles_n = (int)(((long long)N + tile_n - 1) / tile_n);
  const long long tasks = (long long)t.tiles_m * t.tiles_n * split;
  const long long per_xcd = (tasks + 7) / 8;
  t.grid = 8LL * per_xcd;  // the host refuses grids past 2^32 work-items before per_xcd is used
  t.per_xcd = (int)(per_xcd < 0x7FFFFFFF ? per_xcd : 0x7FFFFFFF);
  t.threads = 512;  // eight wavefronts for either width
  t.lds = 0;  // static: the four stages
  const long long KS = ((long long)K + 127) / 128;
  t.sps = (int)(4 * (((KS + split - 1) / split + 3) / 4));
  return t;
}

template <int kTN, int kU>
static const void* tiled_kernel_fn(bool nt_a, bool nt_b) {
  if (nt_a) return nt_b ? reinterpret_cast<const void*>(&gemm_tiled_kernel<kTN, kU, true, true>)
                        : reinterpret_cast<const void*>(&gemm_tiled_kernel<kTN, kU, true, false>);
  return nt_b ? reinterpret_cast<const void*>(&gemm_tiled_kernel<kTN, kU, false, true>)
              : reinterpret_cast<const void*>(&gemm_tiled_kernel<kTN, kU, false, false>);
}

hipError_t launch_gemm_tiled(const uint8_t* a_packed, const uint8_t* b_packed, uint16_t* c, int ldc,
                             int M, int N, int K, int tile_n, int split, float* ws,
                             hipStream_t stream) {
  const TiledGeom t = tiled_geometry(M, N, K, tile_n, split);
  const PackedDims da = packed_dims(M, K), db = packed_dims(N, K);
  TiledArgs args;
  args.ap = a_packed;
  args.bp = b_packed;
  args.c = c;
  args.ws = ws;
  args.split = split;
  args.sps = t.sps;
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
  const bool nt_a = t.tiles_n <= kNtMaxColTiles, nt_b = t.tiles_m <= kNtMaxRowTiles;
  const void* fn = tile_n == 128 ? tiled_kernel_fn<128, 2>(nt_a, nt_b) : tiled_kernel_fn<256, 4>(nt_a, nt_b);
  hipError_t err = hipLaunchKernel(fn, dim3((unsigned)t.grid), dim3(t.threads), kargs, (unsigned)t.lds, stream);
  if (err != hipSuccess) return err;
  if (split > 1) return launch_splitk_reduce(ws, c, M, N, ldc, split, stream);
  return hipSuccess;
}

}  // namespace mx
