// quant.hip -- bf16 -> MXFP4 quantizer kernels and the one-time B repack.
//
// Linear quantizer work unit: one lane takes 8 consecutive bf16 (one
// 16-byte load); the 4 lanes of an aligned quad cover one 32-element group,
// find its maximum with two DPP steps, and each lane encodes its 8 elements
// into one dword of codes.  Loads are coalesced along K (a wave reads 1 KiB
// of contiguous row data).  The packed quantizer instead gives each lane a
// whole group, so that its 16 bytes of codes land in packed order.  Every
// kernel walks its items with a grid-stride loop, so the grid stays within
// a dispatch's 2^32 work-items at any size; the stride is a multiple of
// 256, so quads stay whole.
#include "mx_internal.hpp"

namespace mx {

constexpr int kQuantBlock = 256;
constexpr long long kMaxQuantBlocks = 1 << 20;

// Streaming 16-byte accesses (nontemporal: read or written once, kept out
// of the caches' way; the 8192 x 8192 packed quantization and the B repack
// of 2112 x 7168 ran 17 % and 24 % faster than with plain accesses).
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
    const uint4 v = *reinterpret_cast<const uint4*>(a + (size_t)row * lda + (size_t)kk * 8);
    const uint32_t amax = quad_max(amax8_bits(v));
    const uint32_t byte = scale_byte_from_amax(amax);
    const uint32_t codes = encode8(v, byte);
    *reinterpret_cast<uint32_t*>(out_fp4 + (size_t)row * ld_fp4 + (size_t)kk * 4) = codes;
    if ((kk & 3) == 0) out_scale[(size_t)row * ld_scale + (kk >> 2)] = (uint8_t)byte;
  }
}

// MX-packed output, padding included: rows >= M and K-groups >= K/32 get
// code 0 and scale 127.  One lane per 16-byte chunk of the packed data, in
// packed order (tile t, step j, packed lane l: row 16t + l%16, 32-group
// 4j + l/16), so a wavefront writes one whole 1 KiB block: the lane reads
// its group's 64 bytes, takes the maximum, encodes the 32 values and stores
// the codes, then the group's scale byte into its dword of the scale part.
__global__ __launch_bounds__(kQuantBlock) void quant_packed_kernel(const uint16_t* __restrict__ a, int M,
                                                           int K, int lda,
                                                           uint8_t* __restrict__ out,
                                                           PackedDims d) {
  const long long n_items = (long long)d.RT * d.KS * 64;
  const long long stride = (long long)gridDim.x * blockDim.x;
  const int groups = K / kGroup;
  for (long long it = (long long)blockIdx.x * blockDim.x + threadIdx.x; it < n_items;
       it += stride) {
    const int l = (int)(it & 63);
    const int tj = (int)(it >> 6);  // < 2^31: M*K is at most 2^40
    const int t = tj / d.KS;
    const int j = tj - t * d.KS;
    const int row = 16 * t + (l & 15);
    const int gi = 4 * j + (l >> 4);
    uint4 codes = {0u, 0u, 0u, 0u};
    uint32_t byte = 127;
    if (row < M && gi < groups) {
      const uint4* src = reinterpret_cast<const uint4*>(a + (size_t)row * lda + (size_t)gi * kGroup);
      const uint4 v0 = load_stream16(src), v1 = load_stream16(src + 1);
      const uint4 v2 = load_stream16(src + 2), v3 = load_stream16(src + 3);
      const uint32_t amax = max(max(amax8_bits(v0), amax8_bits(v1)), max(amax8_bits(v2), amax8_bits(v3)));
      byte = scale_byte_from_amax(amax);
      codes = make_uint4(encode8(v0, byte), encode8(v1, byte), encode8(v2, byte), encode8(v3, byte));
    }
    store_stream16(out + (size_t)it * 16, codes);
    uint8_t* sc = out + d.scale_off(t, j >> 2, l);
    sc[j & 3] = (uint8_t)byte;
    if (j == d.KS - 1) {  // fill the unused steps of the last scale dword
      for (int s = (j & 3) + 1; s < 4; ++s) sc[s] = 127;
    }
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
  const long long n = (long long)d.RT * d.KS * 64;
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
