// gemm_stream.hip -- MXFP4 GEMM with pre-quantized A and a K loop inside
// the workgroup, for small M and long K (weights streamed from HBM).
//
// A workgroup of four wavefronts computes all 16*MBW rows of its row group
// against 4 x NTW 16-column tiles of B (one group of NTW tiles per
// wavefront) over a range of K that may be as long as the whole of K.  K
// advances one chunk of four 128-K steps at a time (one scale dword per
// lane).  A chunk's MBW x 4 A blocks and A scale dwords, which all four
// wavefronts multiply, are moved into one stage of a four-stage LDS ring by
// direct global-to-LDS copies; each wavefront's own NTW x 4 B blocks and B
// scale dwords, used by that wavefront alone, are loaded straight into its
// registers (a ring of four register sets).  Both are issued three chunks
// ahead of their use, and every wavefront issues the same number of
// vector-memory instructions per chunk, so one wait on that counter finds a
// chunk complete while the three after it stay in flight.  The products
// are the 16x16x128 block-scaled FP4 instruction of the other GEMM kernel,
// with the same lane map and the same per-lane scale bytes.
//
// Rows past M take scale byte 0 and are never stored; row and column tiles
// past the matrices read the last tile instead and are never stored; steps
// past K read the last step and are multiplied with scale byte 0 on both
// operands, which adds nothing.  With split > 1 each
// workgroup writes an fp32 partial [split][M][N], summed by the reduce
// kernel of gemm.hip.
#include "mx_internal.hpp"

namespace mx {

constexpr int kSWaves = 4;      // wavefronts per workgroup, all along N
constexpr int kSCh = 4;         // 128-K steps per chunk (one scale dword)
constexpr int kSStages = 4;     // ring depth: the chunk being multiplied + three in flight

struct StreamArgs {
  const uint8_t* ap;  // MX-packed A (MT row tiles)
  const uint8_t* bp;  // MX-packed B (NT row tiles)
  uint16_t* c;        // bf16 C [M][ldc]
  float* ws;          // fp32 partials [split][M][N] (split > 1)
  int M, N, ldc;
  int MT, NT, KS, KG;
  int mgroups, ngroups, split;
  int chunks;         // chunks per workgroup (the last workgroup's range may end past K)
};

// B's loads carry the nontemporal hint: each B byte is read once per row
// group and streams through the caches (at 16x16384x16384, 38 us per call
// against 60 us without it; A, which every column group re-reads, keeps
// plain copies).  B goes to registers, not through LDS: each B block feeds
// one wavefront only, and the copy engine's path into LDS moved fewer bytes
// per second than plain loads (the kernel with B staged in LDS took 5-15 %
// longer per call on the weight-streaming shapes).
__device__ inline uint4 ld16_stream(BufRsrc r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCachePolicyNT);
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ inline uint32_t ld4_stream(BufRsrc r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kCachePolicyNT);
}

// LDS bytes of one stage: A data, then A scale dwords.
template <int MBW, int NTW>
struct StreamStage {
  static constexpr int a_data = 0;
  static constexpr int a_scale = MBW * kSCh * kBlockBytes;
  static constexpr int bytes = a_scale + MBW * 256;
  // vector-memory instructions each wavefront issues per chunk: MBW A block
  // copies (the workgroup's MBW*4 split four ways), one A scale block copy
  // (wavefront w takes block w % MBW; with MBW < 4 several wavefronts copy
  // the same bytes to the same place), and the loads of its own NTW*4 B
  // blocks and NTW B scale blocks
  static constexpr int copies = MBW + 1 + 5 * NTW;
};

// Waits until at most N of this wavefront's vector-memory instructions are
// outstanding and its LDS accesses are done, then the workgroup barrier.
// An asm statement: the compiler's barrier would wait for every copy.  (The
// compiler adds its own waits before the uses of the B registers; they ask
// for no more than this one has already ensured.)
template <int N>
__device__ inline void stream_wait_barrier() {
#define MX_STREAM_WAIT(n) \
  if constexpr (N == n) asm volatile("s_waitcnt vmcnt(" #n ")\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  MX_STREAM_WAIT(14)
  MX_STREAM_WAIT(16)
  MX_STREAM_WAIT(20)
  MX_STREAM_WAIT(24)
  MX_STREAM_WAIT(26)
  MX_STREAM_WAIT(30)
#undef MX_STREAM_WAIT
  static_assert(N == 14 || N == 16 || N == 20 || N == 24 || N == 26 || N == 30, "copy counts of the tilings");
}

// The four stages as separate arrays: the compiler tracks the copies into
// each on its own, so a read of one stage waits only for the copies into it.
template <int MBW, int NTW>
__shared__ __align__(16) uint8_t g_sring0[StreamStage<MBW, NTW>::bytes];
template <int MBW, int NTW>
__shared__ __align__(16) uint8_t g_sring1[StreamStage<MBW, NTW>::bytes];
template <int MBW, int NTW>
__shared__ __align__(16) uint8_t g_sring2[StreamStage<MBW, NTW>::bytes];
template <int MBW, int NTW>
__shared__ __align__(16) uint8_t g_sring3[StreamStage<MBW, NTW>::bytes];

template <int MBW, int NTW>
__global__ __launch_bounds__(kSWaves * 64) void gemm_stream_kernel(StreamArgs g) {
  using St = StreamStage<MBW, NTW>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // XCD-aware order, as in gemm_kernel: the row groups of one column task
  // (same B tiles, same K range) get ids equal mod 8, i.e. one XCD.
  const int tasks = g.ngroups * g.split;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int task = xcd + 8 * (slot / g.mgroups);
  if (task >= tasks) return;
  const int mg = slot % g.mgroups;
  const int ng = task % g.ngroups;
  const int s = task / g.ngroups;

  const int m0 = mg * MBW * 16;
  const int chunk0 = s * g.chunks;                        // first chunk of the workgroup
  const int nch = min(g.chunks, g.KG - chunk0);           // chunks that hold steps below K
  const int nt_base = (ng * kSWaves + wave) * NTW;        // first B tile of this wavefront
  const PackedDims da = {g.MT, g.KS, g.KG};
  const PackedDims db = {g.NT, g.KS, g.KG};

  // Copies go through buffer descriptors that cover just this workgroup's
  // tiles (offsets from its first tile fit in 32 bits for K <= 2^22), so an
  // address is a per-lane constant plus a wave-uniform offset; tiles past
  // the operand's last are clamped to it.
  const int t_a0 = mg * MBW, a_tiles = min(MBW, g.MT - t_a0);
  const int t_b0 = ng * kSWaves * NTW, b_tiles = min(kSWaves * NTW, g.NT - t_b0);
  const BufRsrc ra = make_rsrc(g.ap + (size_t)t_a0 * g.KS * kBlockBytes, a_tiles * g.KS * kBlockBytes);
  const BufRsrc rb = make_rsrc(g.bp + (size_t)t_b0 * g.KS * kBlockBytes, b_tiles * g.KS * kBlockBytes);
  const BufRsrc ras = make_rsrc(g.ap + da.data_bytes() + (size_t)t_a0 * g.KG * 256, a_tiles * g.KG * 256);
  const BufRsrc rbs = make_rsrc(g.bp + db.data_bytes() + (size_t)t_b0 * g.KG * 256, b_tiles * g.KG * 256);
  const int lane16 = lane * 16, lane4 = lane * 4;

  // Issue chunk c (0-based within the workgroup): A's copies into LDS stage
  // `stage`, B's loads into the register set bv, bsv.  A chunk past the
  // workgroup's range (issued only to keep the count in flight fixed) reads
  // the same valid 16 (or 4) bytes on every lane: one cache line instead of
  // a chunk of the operands.
  auto issue = [&](int c, uint8_t* stage, uint4 (&bv)[NTW][kSCh], uint32_t (&bsv)[NTW]) {
    const int cg = chunk0 + c;
    const int v16 = c < nch ? lane16 : 0, v4 = c < nch ? lane4 : 0;
#pragma unroll
    for (int i = 0; i < MBW; ++i) {  // A blocks q = wave + 4 i of MBW x 4: block i, step wave
      const int q = wave + kSWaves * i;
      const int b = min(q / kSCh, a_tiles - 1), j = q % kSCh;
      const int step = min(cg * kSCh + j, g.KS - 1);
      dma16(ra, stage + St::a_data + q * kBlockBytes, v16, (b * g.KS + step) * kBlockBytes);
    }
    {
      const int b = min(wave % MBW, a_tiles - 1);
      dma4(ras, stage + St::a_scale + (wave % MBW) * 256, v4, (b * g.KG + min(cg, g.KG - 1)) * 256);
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int slot_b = wave * NTW + i;
      const int lb = min(slot_b, b_tiles - 1);
#pragma unroll
      for (int j = 0; j < kSCh; ++j) {
        const int step = min(cg * kSCh + j, g.KS - 1);
        bv[i][j] = ld16_stream(rb, v16, (lb * g.KS + step) * kBlockBytes);
      }
      bsv[i] = ld4_stream(rbs, v4, (lb * g.KG + min(cg, g.KG - 1)) * 256);
    }
  };

  uint32_t rowmask[MBW];
#pragma unroll
  for (int b = 0; b < MBW; ++b) rowmask[b] = (m0 + b * 16 + (lane & 15)) < g.M ? 0xFFu : 0u;
  f32x4 acc[MBW][NTW];
#pragma unroll
  for (int b = 0; b < MBW; ++b)
#pragma unroll
    for (int i = 0; i < NTW; ++i) acc[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane read offsets inside a stage, each one value (the reads' address
  // chains stay short and separate from the copies' destinations, so the
  // compiler keeps the stage of every read and waits only for that stage's
  // copies).
  const int rd_a = lane * 16;
  const int rd_as = lane * 4;
  // Products of chunk c from LDS stage `stage` and registers bvr, bsr.
  // Steps past K, and every step of chunks past the workgroup's range, take
  // scale byte 0 for both operands: a product of at most 36 * 2^-254, which
  // leaves every fp32 sum unchanged.  No branch: the loop body stays one
  // straight block per stage.
  auto multiply = [&](int c, const uint8_t* stage, const uint4 (&bvr)[NTW][kSCh], const uint32_t (&bsr)[NTW]) {
    const int step0 = (chunk0 + c) * kSCh;
    const uint32_t live = c < nch ? 0xFFu : 0u;
    uint32_t as[MBW], bs[NTW];
#pragma unroll
    for (int b = 0; b < MBW; ++b)
      as[b] = *reinterpret_cast<const uint32_t*>(stage + (rd_as + St::a_scale + b * 256));
#pragma unroll
    for (int i = 0; i < NTW; ++i)
      bs[i] = bsr[i];
#pragma unroll
    for (int j = 0; j < kSCh; ++j) {
      const uint32_t ok = step0 + j < g.KS ? live : 0u;
      uint4 av[MBW], bv[NTW];
#pragma unroll
      for (int b = 0; b < MBW; ++b)
        av[b] = *reinterpret_cast<const uint4*>(stage + (rd_a + St::a_data + (b * kSCh + j) * kBlockBytes));
#pragma unroll
      for (int i = 0; i < NTW; ++i)
        bv[i] = bvr[i][j];
#pragma unroll
      for (int b = 0; b < MBW; ++b) {
        const int asc = (int)((as[b] >> (8 * j)) & rowmask[b] & ok);
#pragma unroll
        for (int i = 0; i < NTW; ++i)
          acc[b][i] = mfma_fp4(av[b], bv[i], acc[b][i], asc, (int)((bs[i] >> (8 * j)) & ok));
      }
    }
  };

  // Chunk c is issued three loop steps before its products, into stage and
  // register set c % 4, unconditionally (chunks past the workgroup's range
  // are never multiplied), so every step has the same instructions in flight
  // and one count waits for exactly chunk c.  The loop runs a multiple of
  // four steps with the stages and register sets named in each.  The
  // scheduling barriers keep the prologue's three chunks in issue order, so
  // the compiler's own count of the loads in flight at the loop head is
  // exact and its waits before B's uses never hold a later chunk.
  constexpr int kC = St::copies;
  uint8_t* const ring0 = g_sring0<MBW, NTW>;
  uint8_t* const ring1 = g_sring1<MBW, NTW>;
  uint8_t* const ring2 = g_sring2<MBW, NTW>;
  uint8_t* const ring3 = g_sring3<MBW, NTW>;
  uint4 b0[NTW][kSCh], b1[NTW][kSCh], b2[NTW][kSCh], b3[NTW][kSCh];
  uint32_t s0[NTW], s1[NTW], s2[NTW], s3[NTW];
  issue(0, ring0, b0, s0);
  __builtin_amdgcn_sched_barrier(0);
  issue(1, ring1, b1, s1);
  __builtin_amdgcn_sched_barrier(0);
  issue(2, ring2, b2, s2);
  __builtin_amdgcn_sched_barrier(0);
  const int nloop = (nch + kSStages - 1) / kSStages * kSStages;
#define MX_STREAM_STEP(R, B, S, R2, B2, S2) \
  stream_wait_barrier<2 * kC>();            \
  issue(c + 3, R2, B2, S2);                 \
  multiply(c, R, B, S);                     \
  ++c;
  for (int c = 0; c < nloop;) {
    MX_STREAM_STEP(ring0, b0, s0, ring3, b3, s3)
    MX_STREAM_STEP(ring1, b1, s1, ring0, b0, s0)
    MX_STREAM_STEP(ring2, b2, s2, ring1, b1, s1)
    MX_STREAM_STEP(ring3, b3, s3, ring2, b2, s2)
  }
#undef MX_STREAM_STEP
  // no copy may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Store: bf16 (nearest even) or an fp32 partial.
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = nt_base + i;
    if (nt >= g.NT) continue;
    const int col = nt * 16 + (lane & 15);
#pragma unroll
    for (int b = 0; b < MBW; ++b) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + b * 16 + 4 * (lane >> 4) + e;
        if (row >= g.M || col >= g.N) continue;
        if (g.split == 1)
          g.c[(size_t)row * g.ldc + col] = f32_to_bf16_rne(acc[b][i][e]);
        else
          g.ws[((size_t)s * g.M + row) * g.N + col] = acc[b][i][e];
      }
    }
  }
}

// ------------------------------------------------------------ host side

#define MX_STREAM_KERNELS(X) X(1, 1) X(1, 2) X(2, 1) X(2, 2) X(4, 1) X(4, 2)

struct StreamEntry {
  int mbw, ntw;
  const void* fn;
  int lds;
};
#define MX_STREAM_ENTRY(MBW, NTW)                                                 \
  {MBW, NTW, reinterpret_cast<const void*>(&gemm_stream_kernel<MBW, NTW>),         \
   kSStages * StreamStage<MBW, NTW>::bytes},
static const StreamEntry kStreamKernels[] = {MX_STREAM_KERNELS(MX_STREAM_ENTRY)};

static const StreamEntry* find_stream(int mbw, int ntw) {
  for (const StreamEntry& e : kStreamKernels)
    if (e.mbw == mbw && e.ntw == ntw) return &e;
  return nullptr;
}

bool stream_kernel_available(int mbw, int ntw) { return find_stream(mbw, ntw) != nullptr; }

StreamGeom stream_geometry(int mbw, int ntw, int steps_per_wg, int M, int N, int K) {
  StreamGeom g;
  const PackedDims d = packed_dims(N, K);
  g.MT = (int)(((long long)M + 15) / 16);
  g.NT = d.RT;
  g.KS = d.KS;
  g.KG = d.KG;
  g.chunks = steps_per_wg / kSCh;
  g.split = (g.KG + g.chunks - 1) / g.chunks;
  g.mgroups = (g.MT + mbw - 1) / mbw;
  g.ngroups = (int)(((long long)g.NT + kSWaves * ntw - 1) / (kSWaves * ntw));
  const long long tasks = (long long)g.ngroups * g.split;
  g.grid = 8LL * ((tasks + 7) / 8) * g.mgroups;
  g.threads = kSWaves * 64;
  const StreamEntry* e = find_stream(mbw, ntw);
  g.lds = e ? e->lds : 0;
  return g;
}

hipError_t launch_gemm_stream(int mbw, int ntw, int steps_per_wg, const uint8_t* a_packed,
                              const uint8_t* b_packed, uint16_t* c, int ldc, int M, int N, int K,
                              float* ws, hipStream_t stream) {
  const StreamEntry* e = find_stream(mbw, ntw);
  if (!e) return hipErrorInvalidDeviceFunction;
  const StreamGeom geo = stream_geometry(mbw, ntw, steps_per_wg, M, N, K);
  StreamArgs args;
  args.ap = a_packed;
  args.bp = b_packed;
  args.c = c;
  args.ws = ws;
  args.M = M;
  args.N = N;
  args.ldc = ldc;
  args.MT = geo.MT;
  args.NT = geo.NT;
  args.KS = geo.KS;
  args.KG = geo.KG;
  args.mgroups = geo.mgroups;
  args.ngroups = geo.ngroups;
  args.split = geo.split;
  args.chunks = geo.chunks;
  void* kargs[] = {&args};
  hipError_t err = hipLaunchKernel(e->fn, dim3((unsigned)geo.grid), dim3(geo.threads), kargs, 0, stream);
  if (err != hipSuccess) return err;
  if (geo.split > 1) return launch_splitk_reduce(ws, c, M, N, ldc, geo.split, stream);
  return hipSuccess;
}

}  // namespace mx
