// gemm.hip -- MXFP4 GEMM kernel (fused or pre-quantized A) and the split-K
// reduce, for gfx950.
//
// Work decomposition (one workgroup):
//   rows    [m0, m0 + 16*MBW)            MBW blocks of the MFMA's 16 rows
//   columns wn wavefronts x NTW tiles of 16 columns
//   K       wk wavefronts x KSW steps of 128, starting at step jw0
// The workgroup's A rows for its K range are staged once in LDS in the
// instruction's lane order -- quantized in the kernel from bf16 (fused
// mode) or copied from the MX-packed A (prequant mode) -- and every
// wavefront reads its A operand from there.  Each wavefront streams its own
// B tiles straight from HBM into registers (16 bytes per lane per step, one
// coalesced 1 KiB block per load instruction); its A loads go first, so the
// A quantization overlaps the B loads' latency.  Partial tiles of the wk
// wavefronts are summed in LDS in a fixed order; with split > 1 the
// workgroup writes an fp32 partial, summed by splitk_reduce_kernel or by the
// last workgroup of the tile.
#include <atomic>

#include "mx_internal.hpp"

namespace mx {

struct GemmArgs {
  const uint16_t* a;  // bf16 A [M][lda] (fused mode)
  const uint8_t* ap;  // MX-packed A (prequant mode)
  const uint8_t* bp;  // MX-packed B
  uint16_t* c;        // bf16 C [M][ldc]
  float* ws;          // fp32 partials [split][M][N], or the [M][N] accumulator (atomic reduce)
  unsigned* counters; // per output tile arrival counters (last-workgroup reduce)
  int M, N, K, lda, ldc;
  int MT, NT, KS, KG;
  int wn, wk, split, mgroups, ngroups, kswg;
  int reduce;          // split > 1: a Reduce value
  unsigned lds_asc_off, lds_red_off;
  unsigned long long kswg_inv;  // floor(2^32 / kswg) + 1: x / kswg == (x * kswg_inv) >> 32
                                // for every x < 2^32 / kswg (33-bit for kswg = 1)
};

// 16-byte load marked nontemporal (streamed, not expected to be re-read soon)
__device__ inline uint4 load_stream16(const void* p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// LDS-direct loads: each active lane moves 16 (or 4) bytes from its own
// global address to lds_base + lane*16 (or lane*4); lds_base must be the
// same for the whole wavefront.
__device__ inline void lds_load16(const void* gptr, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ inline void lds_load4(const void* gptr, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Scale dwords a wavefront's KSW consecutive steps can span.  Step ranges
// start at multiples of KSW, so for KSW % 4 == 0 and KSW <= 2 they never
// straddle more dwords than the step count needs.
template <int KSW>
struct ScaleSpan {
  static constexpr int value = (KSW % 4 == 0) ? KSW / 4 : (KSW <= 2 ? 1 : (KSW + 6) / 4);
};

template <int MODE, int MBW, int NTW, int KSW>
__global__ __launch_bounds__(kMaxThreads) void gemm_kernel(GemmArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr int NSD = ScaleSpan<KSW>::value;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, so everything derived from it lives in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_n = wave % g.wn;
  const int wave_k = wave / g.wn;
  const int nthreads = blockDim.x;

  // XCD-aware order: consecutive workgroup ids go to the 8 XCDs in turn, so
  // workgroup i runs on XCD i % 8.  The mgroups row groups of one column
  // task (same B tiles, same K range) get ids that are equal mod 8 and land
  // on one XCD, where the first read of each B tile fills the L2 for the
  // rest.  The placement only affects speed: every workgroup computes the
  // same thing wherever it runs.  Ids past the last task (padding of the
  // final round) exit at once.
  const int tasks = g.ngroups * g.split;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int task = xcd + 8 * (slot / g.mgroups);
  if (task >= tasks) return;
  const int mg = slot % g.mgroups;
  const int ng = task % g.ngroups;
  const int s = task / g.ngroups;

  const int m0 = mg * MBW * 16;
  const int kswg = g.kswg;
  const int jw0 = s * kswg;             // first K step of the workgroup
  const int j0 = jw0 + wave_k * KSW;    // first K step of this wavefront
  const int gw0 = jw0 >> 2;             // first scale dword of the workgroup
  const int ngw = ((jw0 + kswg - 1) >> 2) - gw0 + 1;
  const int nt_base = (ng * g.wn + wave_n) * NTW;

  // ---- 1. A for steps [jw0, jw0 + kswg).  Fused mode: the first kAPT
  //         chunks of every wavefront are loaded into registers before any B
  //         load is issued (rows past M and chunks past K read the
  //         workgroup's first elements instead, so the number of load
  //         instructions is fixed and the compiler's wait for them leaves the
  //         B loads in flight while A is quantized).  Prequant mode: the
  //         packed A blocks are copied to LDS by LDS-direct loads (global ->
  //         LDS without registers).
  //
  //         Fused A is handled per (row block rg, step jl), numbered
  //         rest = rg*kswg + jl: 16 rows x 128 elements, i.e. four chunks, one
  //         per K-group kg.  In a chunk lane L takes row L/4 and quarter L%4
  //         (8 consecutive bf16, 16 bytes), so an aligned quad of lanes holds
  //         one 32-element group, and the chunk's 64 code dwords fill 64
  //         consecutive LDS words (no bank conflicts).  In load round t,
  //         wavefront w takes rests (t*nwaves + w)*kRestsPerRound + i: every
  //         rest field is wave-uniform (scalar registers) and kg is a
  //         compile-time offset.
  constexpr int kRestsPerRound = kAPT / 4;
  const int nwaves = nthreads >> 6;
  uint8_t* lds_a = smem;
  uint8_t* lds_sc = smem + g.lds_asc_off;
  const int rows_valid = min(MBW * 16, g.M - m0);
  const int n_rests = MODE == 1 ? ((rows_valid + 15) >> 4) * kswg : 0;
  const int groups = g.K / kGroup;
  const int r16 = lane >> 2;
  struct Rest {
    int rg, jl;
    bool live;    // rest < n_rests: its LDS slots exist
    int kg_end;   // K-groups kg < kg_end lie below K (<= 0 when not live)
    bool row_ok;  // per lane: the lane's row is below M
  };
  auto rest_info = [&](int rest) {
    Rest x;
    x.rg = MBW == 1 ? 0 : (int)(((unsigned long long)rest * g.kswg_inv) >> 32);
    x.jl = rest - x.rg * kswg;
    x.live = rest < n_rests;
    x.kg_end = x.live ? groups - (jw0 + x.jl) * 4 : 0;
    x.row_ok = r16 < rows_valid - x.rg * 16;
    return x;
  };
  const uint16_t* a_first = g.a + (size_t)m0 * g.lda + (size_t)jw0 * kStep;
  const size_t a_lane = (size_t)r16 * g.lda + (lane & 3) * 8;
  auto load_rest = [&](const Rest& x, uint4* v) {
    const uint16_t* base = a_first + (size_t)x.rg * 16 * g.lda + (size_t)x.jl * kStep;
    const size_t lane_off = x.row_ok ? a_lane : (size_t)(lane & 3) * 8;
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint16_t* src = (kg < x.kg_end ? base + kg * kGroup : a_first) + lane_off;
      v[kg] = *reinterpret_cast<const uint4*>(src);
    }
  };
  auto quantize_rest = [&](int rest, const Rest& x, const uint4* v) {
    if (!x.live || !x.row_ok) return;
    const int jj = jw0 + x.jl;
    uint8_t* codes_at = lds_a + (size_t)rest * kBlockBytes + 4 * lane;
    uint8_t* scale_at = lds_sc + ((size_t)(x.rg * ngw + (jj >> 2) - gw0) * 64 + r16) * 4 + (jj & 3);
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      // groups past K are quantized as zeros: zero magnitudes, zero codes
      const bool in = kg < x.kg_end;
      const uint32_t amax = quad_max(amax8_bits(v[kg], in ? 0x7FFF7FFFu : 0u));
      const uint32_t byte = scale_byte_from_amax(amax);
      const uint32_t codes = encode8(v[kg], byte);
      *reinterpret_cast<uint32_t*>(codes_at + kg * 256) = in ? codes : 0u;
      if ((lane & 3) == 0) scale_at[kg * 64] = (uint8_t)byte;
    }
  };
  uint4 araw[kAPT];
  if constexpr (MODE == 1) {
    // Rests past the first round (plans whose A stage exceeds kAPT chunks
    // per wavefront) are loaded and quantized first, round by round, so that
    // no load is ever issued after the B loads: a load younger than B would
    // make every later wait for it a wait for all of B.
    for (int r0 = (nwaves + wave) * kRestsPerRound; r0 < n_rests; r0 += nwaves * kRestsPerRound) {
#pragma unroll
      for (int i = 0; i < kRestsPerRound; ++i) load_rest(rest_info(r0 + i), araw + 4 * i);
#pragma unroll
      for (int i = 0; i < kRestsPerRound; ++i) quantize_rest(r0 + i, rest_info(r0 + i), araw + 4 * i);
    }
#pragma unroll
    for (int i = 0; i < kRestsPerRound; ++i)
      load_rest(rest_info(wave * kRestsPerRound + i), araw + 4 * i);
  } else {
    const PackedDims da = {g.MT, g.KS, g.KG};
    const int mbv = min(MBW, g.MT - mg * MBW);
    const int n_blocks = mbv * kswg;
    for (int bi = wave; bi < n_blocks; bi += nwaves) {
      const int b = bi / kswg;
      const int jl = bi - b * kswg;
      lds_load16(g.ap + da.data_off(mg * MBW + b, jw0 + jl, lane),
                 lds_a + (size_t)(b * kswg + jl) * 1024);
    }
    const int n_sd = mbv * ngw;
    for (int bi = wave; bi < n_sd; bi += nwaves) {
      const int b = bi / ngw;
      const int gl = bi - b * ngw;
      lds_load4(g.ap + da.scale_off(mg * MBW + b, gw0 + gl, lane),
                lds_sc + (size_t)(b * ngw + gl) * 256);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. issue every B load of this wavefront (clamped tile index keeps a
  //         ragged last group in bounds; its results are never stored).
  //         Nontemporal: B streams from HBM, and the row groups that share
  //         a tile read it at about the same time (10 % faster at
  //         M=16, K=7168, 6 % at M=64 than plain loads; the same marking
  //         on A, which every column group re-reads, was slower).
  uint4 bq[NTW][KSW];
  uint32_t bs[NTW][NSD];
  const size_t b_sc_base = (size_t)g.NT * g.KS * kBlockBytes;
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = min(nt_base + i, g.NT - 1);
    const uint8_t* bt = g.bp + ((size_t)nt * g.KS + j0) * kBlockBytes + (size_t)lane * 16;
#pragma unroll
    for (int j = 0; j < KSW; ++j) bq[i][j] = load_stream16(bt + (size_t)j * kBlockBytes);
    const uint8_t* bst = g.bp + b_sc_base + (size_t)nt * g.KG * 256 + (size_t)lane * 4;
#pragma unroll
    for (int d = 0; d < NSD; ++d) {
      const int gi = min((j0 >> 2) + d, g.KG - 1);
      bs[i][d] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(bst + (size_t)gi * 256));
    }
  }

  if constexpr (MODE == 1) {
#pragma unroll
    for (int i = 0; i < kRestsPerRound; ++i) {
      const int rest = wave * kRestsPerRound + i;
      quantize_rest(rest, rest_info(rest), araw + 4 * i);
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0);  // the LDS-direct copies
  }
  __syncthreads();

  // ---- 3. block-scaled FP4 products.  Rows >= M get scale byte 0 and are
  //         never stored.  The wavefront's A scale dwords are read from LDS
  //         once; A codes are read kAhead steps ahead of their product.
  constexpr int kAhead = MBW >= 4 ? 2 : 3;  // LDS reads in flight stay within the wait counter
  uint32_t rowmask[MBW];
#pragma unroll
  for (int b = 0; b < MBW; ++b) rowmask[b] = (m0 + b * 16 + (lane & 15)) < g.M ? 0xFFu : 0u;

  f32x4 acc[MBW][NTW];
#pragma unroll
  for (int b = 0; b < MBW; ++b)
#pragma unroll
    for (int i = 0; i < NTW; ++i) acc[b][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t as[MBW][NSD];
#pragma unroll
  for (int b = 0; b < MBW; ++b)
#pragma unroll
    for (int d = 0; d < NSD; ++d) {
      const int rel = min((j0 >> 2) + d - gw0, ngw - 1);
      as[b][d] = *reinterpret_cast<const uint32_t*>(lds_sc + ((size_t)(b * ngw + rel) * 64 + lane) * 4);
    }
  uint4 av[KSW][MBW];  // statically indexed: only kAhead + 2 steps are live at once
  auto read_a = [&](int j) {
    const int jl = wave_k * KSW + j;
#pragma unroll
    for (int b = 0; b < MBW; ++b)
      av[j][b] = *reinterpret_cast<const uint4*>(lds_a + ((size_t)(b * kswg + jl) * 64 + lane) * 16);
  };
#pragma unroll
  for (int j = 0; j <= kAhead && j < KSW; ++j) read_a(j);

#pragma unroll
  for (int j = 0; j < KSW; ++j) {
    if (j + kAhead + 1 < KSW) read_a(j + kAhead + 1);
    // keep the later steps' LDS reads ahead of this step's products
    __builtin_amdgcn_sched_barrier(0);
    // Scale bytes of step j: dword d of as/bs holds steps 4*((j0 >> 2) + d)
    // .. +3, one byte each.  Where that dword is not known at compile time
    // it is chosen by selects (an indexed access would move the arrays to
    // scratch memory).
    const int jj = j0 + j;
    const int sh = (KSW % 4 == 0) ? 8 * (j & 3) : 8 * (jj & 3);
    constexpr bool kStatic = KSW % 4 == 0 || KSW <= 2;
    const int dsel = kStatic ? ((KSW % 4 == 0) ? (j >> 2) : 0) : (jj >> 2) - (j0 >> 2);
    int bsc[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      uint32_t w = bs[i][0];
#pragma unroll
      for (int d = 1; d < NSD; ++d) w = (dsel == d) ? bs[i][d] : w;
      bsc[i] = (int)((w >> sh) & 0xFFu);
    }
#pragma unroll
    for (int b = 0; b < MBW; ++b) {
      uint32_t w = as[b][0];
#pragma unroll
      for (int d = 1; d < NSD; ++d) w = (dsel == d) ? as[b][d] : w;
      const int asc = (int)((w >> sh) & rowmask[b]);
#pragma unroll
      for (int i = 0; i < NTW; ++i) acc[b][i] = mfma_fp4(av[j][b], bq[i][j], acc[b][i], asc, bsc[i]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 4. sum the wk wavefronts of one column group in LDS, in order.
  //         Every wavefront stays to the end so that each barrier below is
  //         reached by the whole workgroup; only wave_k == 0 stores.
  const bool owner = wave_k == 0;
  if (g.wk > 1) {
    float* red = reinterpret_cast<float*>(smem + g.lds_red_off);
    constexpr int per_wave = MBW * NTW * 256;
    if (!owner) {
      float* dst = red + (size_t)((wave_k - 1) * g.wn + wave_n) * per_wave;
#pragma unroll
      for (int b = 0; b < MBW; ++b)
#pragma unroll
        for (int i = 0; i < NTW; ++i)
          *reinterpret_cast<f32x4*>(dst + ((b * NTW + i) * 64 + lane) * 4) = acc[b][i];
    }
    __syncthreads();
    if (owner) {
      for (int kk = 1; kk < g.wk; ++kk) {
        const float* src = red + (size_t)((kk - 1) * g.wn + wave_n) * per_wave;
#pragma unroll
        for (int b = 0; b < MBW; ++b)
#pragma unroll
          for (int i = 0; i < NTW; ++i)
            acc[b][i] += *reinterpret_cast<const f32x4*>(src + ((b * NTW + i) * 64 + lane) * 4);
      }
    }
  }

  // ---- 5. store: bf16 (nearest even) or an fp32 partial.
  if (owner) {
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
          float* part = g.ws + ((size_t)s * g.M + row) * g.N + col;
          if (g.split == 1)
            g.c[(size_t)row * g.ldc + col] = f32_to_bf16_rne(acc[b][i][e]);
          else if (g.reduce == kReduceAtomic)
            __hip_atomic_fetch_add(g.ws + (size_t)row * g.N + col, acc[b][i][e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          else if (g.reduce == kReduceLastWg)
            __hip_atomic_store(part, acc[b][i][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            *part = acc[b][i][e];
        }
      }
    }
  }
  if (g.split == 1 || g.reduce == kReduceKernel) return;

  // ---- 6. split-K finished by the last workgroup of this output tile.
  //         The partials above are agent-scope atomic stores (or, for the
  //         atomic reduce, agent-scope atomic adds into one accumulator).
  //         Ordering, in the HIP memory model: the barrier orders every
  //         thread's partial stores before thread 0's increment of the tile
  //         counter, an acquire-release read-modify-write at agent scope (on
  //         gfx950: an L2 write-back before it, an invalidate after it).  The
  //         workgroup whose increment takes the counter to split-1 has
  //         therefore acquired every other workgroup's release, and its
  //         second barrier passes that on to all of its threads, which then
  //         read the partials.  Last-workgroup reduce: the partials are
  //         summed in order s = 0..split-1 (the order of
  //         splitk_reduce_kernel, so both give identical bits).  Atomic
  //         reduce: the accumulator already holds the sum (its order of
  //         additions varies from call to call) and is cleared again.  The
  //         counter returns to zero for the next call on this workspace (a
  //         later launch, ordered by the kernel boundary).  The flag lives in
  //         the first LDS word: every LDS read above is behind the first
  //         barrier here.
  volatile int* is_last = reinterpret_cast<volatile int*>(smem);
  __builtin_amdgcn_s_waitcnt(0);  // every wavefront's stores have completed at the barrier
  __syncthreads();
  const int tile = mg * g.ngroups + ng;
  if (tid == 0) {
    const unsigned old =
        __hip_atomic_fetch_add(g.counters + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *is_last = (old == (unsigned)(g.split - 1));
  }
  __syncthreads();
  if (!*is_last) return;
  if (owner && g.reduce == kReduceAtomic) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = nt_base + i;
      if (nt >= g.NT) continue;
      const int col = nt * 16 + (lane & 15);
#pragma unroll
      for (int b = 0; b < MBW; ++b) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + b * 16 + 4 * (lane >> 4) + e;
          if (row < g.M && col < g.N)
            v[e] = __hip_atomic_load(g.ws + (size_t)row * g.N + col, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + b * 16 + 4 * (lane >> 4) + e;
          if (row < g.M && col < g.N) {
            g.c[(size_t)row * g.ldc + col] = f32_to_bf16_rne(v[e]);
            __hip_atomic_store(g.ws + (size_t)row * g.N + col, 0.0f, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  } else if (owner) {
    const size_t plane = (size_t)g.M * g.N;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = nt_base + i;
      if (nt >= g.NT) continue;
      const int col = nt * 16 + (lane & 15);
#pragma unroll
      for (int b = 0; b < MBW; ++b) {
        // all split partials of this lane's 4 outputs are requested before
        // the first is summed (rows >= M read row 0 and are not stored)
        float v[4][kMaxLastWgSplit];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = min(m0 + b * 16 + 4 * (lane >> 4) + e, g.M - 1);
          float* src = g.ws + (size_t)row * g.N + min(col, g.N - 1);
#pragma unroll
          for (int k = 0; k < kMaxLastWgSplit; ++k)
            if (k < g.split)
              v[e][k] = __hip_atomic_load(src + (size_t)k * plane, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + b * 16 + 4 * (lane >> 4) + e;
          float sum = v[e][0];
#pragma unroll
          for (int k = 1; k < kMaxLastWgSplit; ++k)
            if (k < g.split) sum += v[e][k];
          if (row < g.M && col < g.N) g.c[(size_t)row * g.ldc + col] = f32_to_bf16_rne(sum);
        }
      }
    }
  }
  if (tid == 0) __hip_atomic_store(g.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum split fp32 partials [S][M][N] in order s = 0..S-1 and round to bf16.
// With N % 4 == 0 one thread takes 4 consecutive outputs (16-byte loads);
// otherwise one output.  The partials are loaded kRedChunk at a time, all of
// a chunk requested before the first is added; one wavefront per workgroup
// spreads the small grid over many CUs.
constexpr int kRedChunk = 8;
constexpr int kRedThreads = 64;

template <typename V, typename Add>
__device__ inline V sum_partials(const V* src, size_t plane, int S, Add add) {
  V acc{};
  for (int k0 = 0; k0 < S; k0 += kRedChunk) {
    V v[kRedChunk];
#pragma unroll
    for (int u = 0; u < kRedChunk; ++u)
      if (k0 + u < S) v[u] = src[(size_t)(k0 + u) * plane];
#pragma unroll
    for (int u = 0; u < kRedChunk; ++u)
      if (k0 + u < S) acc = (k0 + u == 0) ? v[u] : add(acc, v[u]);
  }
  return acc;
}

__global__ __launch_bounds__(kRedThreads) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                                    uint16_t* __restrict__ c,
                                                                    int M, int N, int ldc, int S) {
  const size_t plane = (size_t)M * N;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if ((N & 3) != 0) {
    if (idx >= (long long)plane) return;
    const int row = (int)(idx / N);
    const int col = (int)(idx % N);
    const float acc = sum_partials(ws + idx, plane, S, [](float a, float b) { return a + b; });
    c[(size_t)row * ldc + col] = f32_to_bf16_rne(acc);
    return;
  }
  const int n4 = N / 4;
  if (idx >= (long long)M * n4) return;
  const int row = (int)(idx / n4);
  const int col = (int)(idx % n4) * 4;
  const float4 acc = sum_partials(reinterpret_cast<const float4*>(ws + (size_t)row * N + col),
                                  plane / 4, S, [](float4 a, float4 b) {
                                    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
                                  });
  uint16_t* dst = c + (size_t)row * ldc + col;
  const uint16_t h0 = f32_to_bf16_rne(acc.x), h1 = f32_to_bf16_rne(acc.y);
  const uint16_t h2 = f32_to_bf16_rne(acc.z), h3 = f32_to_bf16_rne(acc.w);
  if ((((uintptr_t)dst) & 7) == 0) {
    uint2 pk;
    pk.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
    pk.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
    *reinterpret_cast<uint2*>(dst) = pk;
  } else {
    dst[0] = h0;
    dst[1] = h1;
    dst[2] = h2;
    dst[3] = h3;
  }
}

// Zero-fill of a scratch prefix by plain vector stores (a fill kernel rather
// than a memset node, so that a captured call replays it correctly).
__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* p, unsigned long long words) {
  const unsigned long long stride = (unsigned long long)gridDim.x * blockDim.x;
  for (unsigned long long i = (unsigned long long)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += stride)
    p[i] = 0u;
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const unsigned long long words = bytes / 4;
  const unsigned long long blocks = (words + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 4096 ? (blocks ? blocks : 1) : 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

// ------------------------------------------------------------ dispatch table

#define MX_KSW_LIST(X, MODE, MBW, NTW) \
  X(MODE, MBW, NTW, 1)                 \
  X(MODE, MBW, NTW, 2)                 \
  X(MODE, MBW, NTW, 3)                 \
  X(MODE, MBW, NTW, 4)                 \
  X(MODE, MBW, NTW, 6)                 \
  X(MODE, MBW, NTW, 7)                 \
  X(MODE, MBW, NTW, 8)                 \
  X(MODE, MBW, NTW, 12)                \
  X(MODE, MBW, NTW, 14)                \
  X(MODE, MBW, NTW, 16)

#define MX_NTW_LIST(X, MODE, MBW) \
  MX_KSW_LIST(X, MODE, MBW, 1)    \
  MX_KSW_LIST(X, MODE, MBW, 2)

#define MX_MBW_LIST(X, MODE) \
  MX_NTW_LIST(X, MODE, 1)    \
  MX_NTW_LIST(X, MODE, 2)    \
  MX_NTW_LIST(X, MODE, 4)

#define MX_ALL_KERNELS(X) \
  MX_MBW_LIST(X, 1)       \
  MX_MBW_LIST(X, 2)

struct KernelEntry {
  int mode, mbw, ntw, ksw;
  const void* fn;
};

#define MX_ENTRY(MODE, MBW, NTW, KSW) \
  {MODE, MBW, NTW, KSW, reinterpret_cast<const void*>(&gemm_kernel<MODE, MBW, NTW, KSW>)},

static const KernelEntry kKernels[] = {MX_ALL_KERNELS(MX_ENTRY)};
constexpr int kNumKernels = sizeof(kKernels) / sizeof(kKernels[0]);
// Kernels whose LDS exceeds 64 KiB need the dynamic-LDS limit raised once per
// device (the attribute belongs to the function on the current device);
// devices past kAttrDevices raise it on every such launch.
constexpr int kAttrDevices = 64;
static std::atomic<int> g_lds_attr_set[kAttrDevices][kNumKernels];

static int find_kernel(int mode, int mbw, int ntw, int ksw) {
  for (int i = 0; i < kNumKernels; ++i)
    if (kKernels[i].mode == mode && kKernels[i].mbw == mbw && kKernels[i].ntw == ntw &&
        kKernels[i].ksw == ksw)
      return i;
  return -1;
}

bool gemm_kernel_available(int mode, int mbw, int ntw, int ksw) {
  return find_kernel(mode, mbw, ntw, ksw) >= 0;
}

GemmGeom gemm_geometry(const Plan& p, int M, int N, int K) {
  GemmGeom g;
  const PackedDims bd = packed_dims(N, K);
  g.MT = (int)(((long long)M + 15) / 16);
  g.NT = bd.RT;
  g.KS = bd.KS;
  g.KG = bd.KG;
  g.mgroups = (int)(((long long)g.MT + p.mbw - 1) / p.mbw);
  const int cols_per_wg = p.wn * p.ntw;
  g.ngroups = (int)(((long long)g.NT + cols_per_wg - 1) / cols_per_wg);
  g.kswg = p.wk * p.ksw;
  g.ngw_max = (g.kswg % 4 == 0) ? g.kswg / 4 : (g.kswg + 6) / 4;
  g.lds_a = (size_t)p.mbw * g.kswg * kBlockBytes;
  g.lds_asc = (size_t)p.mbw * g.ngw_max * 256;
  g.lds_red = p.wk > 1 ? (size_t)(p.wk - 1) * p.wn * p.mbw * p.ntw * 1024 : 0;
  g.lds_total = g.lds_a + g.lds_asc + g.lds_red;
  const long long tasks = (long long)g.ngroups * p.split;
  g.grid = (unsigned)(8 * ((tasks + 7) / 8) * g.mgroups);
  g.threads = p.wn * p.wk * 64;
  return g;
}

hipError_t launch_gemm(const Plan& p, const void* a, int lda, const uint8_t* b_packed,
                       uint16_t* c, int ldc, int M, int N, int K, float* ws,
                       unsigned* counters, hipStream_t stream) {
  const int ki = find_kernel(p.mode, p.mbw, p.ntw, p.ksw);
  if (ki < 0) return hipErrorInvalidDeviceFunction;
  const GemmGeom geo = gemm_geometry(p, M, N, K);
  const void* fn = kKernels[ki].fn;
  if (geo.lds_total > 64 * 1024) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool cached = dev >= 0 && dev < kAttrDevices;
    if (!cached || !g_lds_attr_set[dev][ki].load(std::memory_order_acquire)) {
      e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
      if (e != hipSuccess) return e;
      if (cached) g_lds_attr_set[dev][ki].store(1, std::memory_order_release);
    }
  }
  GemmArgs args;
  args.a = p.mode == 1 ? static_cast<const uint16_t*>(a) : nullptr;
  args.ap = p.mode == 2 ? static_cast<const uint8_t*>(a) : nullptr;
  args.bp = b_packed;
  args.c = c;
  args.ws = ws;
  args.counters = counters;
  args.reduce = p.split > 1 ? p.reduce : kReduceKernel;
  args.M = M;
  args.N = N;
  args.K = K;
  args.lda = lda;
  args.ldc = ldc;
  args.MT = geo.MT;
  args.NT = geo.NT;
  args.KS = geo.KS;
  args.KG = geo.KG;
  args.wn = p.wn;
  args.wk = p.wk;
  args.split = p.split;
  args.mgroups = geo.mgroups;
  args.ngroups = geo.ngroups;
  args.kswg = geo.kswg;
  args.lds_asc_off = (unsigned)geo.lds_a;
  args.lds_red_off = (unsigned)(geo.lds_a + geo.lds_asc);
  args.kswg_inv = (1ull << 32) / (unsigned long long)geo.kswg + 1;
  void* kargs[] = {&args};
  hipError_t e = hipLaunchKernel(fn, dim3(geo.grid), dim3(geo.threads), kargs,
                                 (unsigned)geo.lds_total, stream);
  if (e != hipSuccess) return e;
  if (p.split > 1 && p.reduce == kReduceKernel) e = launch_splitk_reduce(ws, c, M, N, ldc, p.split, stream);
  return e;
}

hipError_t launch_splitk_reduce(const float* ws, uint16_t* c, int M, int N, int ldc, int S,
                                hipStream_t stream) {
  const long long n = (N % 4 == 0) ? (long long)M * (N / 4) : (long long)M * N;
  const unsigned grid = (unsigned)((n + kRedThreads - 1) / kRedThreads);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid), dim3(kRedThreads), 0, stream, ws, c, M, N, ldc, S);
  return hipGetLastError();
}

}  // namespace mx
