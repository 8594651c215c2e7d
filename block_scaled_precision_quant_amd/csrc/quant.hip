// quant.hip -- bf16 -> MXFP4 quantizer kernels and the one-time B repack.
//
// Linear quantizer work unit: one lane takes 8 consecutive bf16 (one
// 16-byte load); the 4 lanes of an aligned quad cover one 32-element group,
// find its maximum with two DPP steps, and each lane encodes its 8 elements
// into one dword of codes.  Loads are coalesced along K (a wave reads 1 KiB
// of contiguous row data).  The packed quantizer reads the same way, four
// rows per load, and stores each dword at its place in the packed order.
// Every kernel walks its items with a grid-stride loop, so the grid stays
// within a dispatch's 2^32 work-items at any size; the stride is a multiple
// of 256 threads, so quads and wavefronts stay whole.
#include "mx_internal.hpp"

namespace mx {

constexpr int kQuantBlock = 256;
constexpr long long kMaxQuantBlocks = 1 << 20;

// Streaming 16-byte accesses (nontemporal: read or written once, kept out
// of the caches' way).  With nontemporal loads the 8192 x 8192 packed
// quantization takes 33 us against 54 us, the linear one 36 us against
// 52 us; the B repack of 2112 x 7168 ran 24 % faster.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store_stream16(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

// Linear output: fp4 [M][ld_fp4] and e8m0 [M][ld_scale].
__global__ __launch_bounds__(kQuantBlock) void quant_linear_kernel(const uint16_t* __restrict__ a, int M,
                                                           int K, int lda,
                                                           uint8_t* __restrict__ out_fp4,
                                                           int ld_fp4,
                                                           uint8_t* __restrict__ out_scale,
                                                           int ld_scale) {
  const int per_row = K / 8;  // 8-element items per row (multiple of 4)
  const long long n_items = (long long)M * per_row;
  const long long stride = (long long)gridDim.x * blockDim.x;
  // n_items is a multiple of 4 and the block size of 256 keeps quads
  // aligned, so a quad is either wholly in range or wholly out.
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < n_items;
       it += stride) {
    const int row = (int)(it / per_row);
    const int kk = (int)(it % per_row);
    const uint4 v = load_stream16(a + (size_t)row * lda + (size_t)kk * 8);
    const uint32_t amax = quad_max(amax8_bits(v));
    const uint32_t byte = scale_byte_from_amax(amax);
    const uint32_t codes = encode8(v, byte);
    *reinterpret_cast<uint32_t*>(out_fp4 + (size_t)row * ld_fp4 + (size_t)kk * 4) = codes;
    if ((kk & 3) == 0) out_scale[(size_t)row * ld_scale + (kk >> 2)] = (uint8_t)byte;
  }
}

// MX-packed output, padding included: rows >= M and K-groups >= K/32 get
// code 0 and scale 127.  One wavefront per (tile t, scale dword g4, row
// quarter q): rows 16t + 4q .. 16t + 4q + 3 over the four 128-K steps whose
// scale bytes share a dword.  For step s, lane l reads 8 bf16 of row
// 16t + 4q + l/16 at K offset 128 (4 g4 + s) + 8 (l%16), so each quarter of
// the wavefront reads one row's 256 contiguous bytes.  The four lanes of an
// aligned quad hold one 32-group (group l%16/4 of the step): two DPP steps
// give its maximum, and each lane encodes its 8 values into the dword l%4 of
// packed lane L = 4q + l/16 + 16 (l%16/4).  The quad's first lane gathers
// the group's four scale bytes and writes the scale dword whole.
__global__ __launch_bounds__(kQuantBlock) void quant_packed_kernel(const uint16_t* __restrict__ a, int M,
                                                           int K, int lda,
                                                           uint8_t* __restrict__ out,
                                                           PackedDims d) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 3, gq = (lane >> 2) & 3, rq = lane >> 4;
  const int groups = K / kGroup;
  const long long n_items = (long long)d.RT * d.KG * 4;
  const long long stride = (long long)gridDim.x * (kQuantBlock / 64);
  for (long long w = (long long)blockIdx.x * (kQuantBlock / 64) + (threadIdx.x >> 6); w < n_items;
       w += stride) {
    const int q = (int)(w & 3);
    const long long tg = w >> 2;
    const int t = (int)(tg / d.KG);
    const int g4 = (int)(tg - (long long)t * d.KG);
    const int row = 16 * t + 4 * q + rq;
    const int L = 4 * q + rq + 16 * gq;
    const int nsteps = min(4, d.KS - 4 * g4);
    const uint16_t* src = a + (size_t)min(row, M - 1) * lda + (size_t)g4 * (4 * kStep) + 8 * (lane & 15);
    uint4 v[4];
    bool valid[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      valid[s] = s < nsteps && row < M && 4 * (4 * g4 + s) + gq < groups;
      v[s] = valid[s] ? load_stream16(src + s * kStep) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t word = 0x7F7F7F7Fu;  // steps past the last keep scale 127
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < nsteps) {  // wave-uniform
        const uint32_t amax = quad_max(amax8_bits(v[s]));
        const uint32_t byte = valid[s] ? scale_byte_from_amax(amax) : 127u;
        const uint32_t codes = valid[s] ? encode8(v[s], byte) : 0u;
        __builtin_nontemporal_store(codes, reinterpret_cast<uint32_t*>(out + d.data_off(t, 4 * g4 + s, L) + 4 * sub));
        word = (word & ~(0xFFu << (8 * s))) | (byte << (8 * s));
      }
    }
    if (sub == 0) *reinterpret_cast<uint32_t*>(out + d.scale_off(t, g4, L)) = word;
  }
}

// One-time repack of linear fp4 [N][K/2] + e8m0 [N][K/32] into MX-packed.
// Threads [0, RT*KS*64) move one 16-byte data chunk each; threads
// [RT*KS*64, RT*KS*64 + RT*KG*64) assemble one scale dword each.  Rows >= N
// and K beyond K get code 0 and scale 127.
__global__ __launch_bounds__(kQuantBlock) void pack_b_kernel(const uint8_t* __restrict__ b_fp4,
                                                     const uint8_t* __restrict__ b_scale, int N,
                                                     int K, uint8_t* __restrict__ out,
                                                     PackedDims d) {
  const long long n_data = (long long)d.RT * d.KS * 64;
  const long long n_scale = (long long)d.RT * d.KG * 64;
  const int groups = K / kGroup;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < n_data + n_scale;
       it += stride) {
    if (it < n_data) {
      const int lane = (int)(it & 63);
      const long long tj = it >> 6;
      const int j = (int)(tj % d.KS);
      const int t = (int)(tj / d.KS);
      const int row = 16 * t + (lane & 15);
      const int g = 4 * j + (lane >> 4);  // the 32-group this lane's 16 bytes hold
      uint4 v = {0u, 0u, 0u, 0u};
      if (row < N && g < groups) v = load_stream16(b_fp4 + (size_t)row * (K / 2) + (size_t)g * 16);
      store_stream16(out + d.data_off(t, j, lane), v);
      continue;
    }
    const long long is = it - n_data;
    const int lane = (int)(is & 63);
    const long long tg = is >> 6;
    const int g4 = (int)(tg % d.KG);
    const int t = (int)(tg / d.KG);
    const int row = 16 * t + (lane & 15);
    uint32_t word = 0;
    for (int s = 0; s < 4; ++s) {
      const int grp = 4 * (4 * g4 + s) + (lane >> 4);
      const uint32_t byte =
          (row < N && grp < groups) ? b_scale[(size_t)row * groups + grp] : 127u;
      word |= byte << (8 * s);
    }
    *reinterpret_cast<uint32_t*>(out + d.scale_off(t, g4, lane)) = word;
  }
}

// --------------------------------------------------------------- launchers

// blocks for `threads` items: one item per thread up to kMaxQuantBlocks
// blocks, more per thread (grid-stride) beyond
static inline unsigned grid_for(long long threads) {
  const long long blocks = (threads + kQuantBlock - 1) / kQuantBlock;
  return (unsigned)(blocks < kMaxQuantBlocks ? blocks : kMaxQuantBlocks);
}

void launch_quant_linear(const uint16_t* a, int M, int K, int lda, uint8_t* out_fp4, int ld_fp4,
                         uint8_t* out_scale, int ld_scale, hipStream_t stream) {
  const long long n = (long long)M * (K / 8);
  hipLaunchKernelGGL(quant_linear_kernel, dim3(grid_for(n)), dim3(kQuantBlock), 0, stream, a, M, K,
                     lda, out_fp4, ld_fp4, out_scale, ld_scale);
}

void launch_quant_packed(const uint16_t* a, int M, int K, int lda, uint8_t* out,
                         hipStream_t stream) {
  const PackedDims d = packed_dims(M, K);
  const long long n = (long long)d.RT * d.KG * 4 * 64;  // one wavefront per item
  hipLaunchKernelGGL(quant_packed_kernel, dim3(grid_for(n)), dim3(kQuantBlock), 0, stream, a, M, K,
                     lda, out, d);
}

void launch_pack_b(const uint8_t* b_fp4, const uint8_t* b_scale, int N, int K, uint8_t* out,
                   hipStream_t stream) {
  const PackedDims d = packed_dims(N, K);
  const long long n = (long long)d.RT * d.KS * 64 + (long long)d.RT * d.KG * 64;
  hipLaunchKernelGGL(pack_b_kernel, dim3(grid_for(n)), dim3(kQuantBlock), 0, stream, b_fp4, b_scale,
                     N, K, out, d);
}

}  // namespace mx
