// mx_device.hpp -- gfx950 device helpers shared by the MXFP4 kernels:
// MX-packed layout offsets, the group scale rule, the e2m1 encoder and the
// block-scaled FP4 matrix instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 32;        // K-elements per e8m0 scale
constexpr int kStep = 128;        // K-elements per matrix instruction
constexpr int kTileRows = 16;     // rows per packed tile
constexpr int kBlockBytes = 1024; // one (tile, step) data block: 64 lanes x 16 B

// ---------------------------------------------------------------- layout
// MX-packed layout of R rows x K columns (see mxfp4.h for the closed form).
struct PackedDims {
  int RT;  // row tiles
  int KS;  // 128-K steps
  int KG;  // scale dwords per (tile, lane): ceil(KS/4)
  __host__ __device__ size_t data_bytes() const { return (size_t)RT * KS * kBlockBytes; }
  __host__ __device__ size_t total_bytes() const { return data_bytes() + (size_t)RT * KG * 256; }
  __host__ __device__ size_t data_off(int t, int j, int lane) const {
    return (((size_t)t * KS + j) * 64 + lane) * 16;
  }
  __host__ __device__ size_t scale_off(int t, int g, int lane) const {
    return data_bytes() + (((size_t)t * KG + g) * 64 + lane) * 4;
  }
};

// K is padded up to whole 128-element steps; the padding holds code 0 and
// scale 127 (a zero contribution).
__host__ __device__ inline PackedDims packed_dims(int rows, int K) {
  PackedDims d;
  d.RT = (int)(((long long)rows + kTileRows - 1) / kTileRows);  // no overflow near INT_MAX
  d.KS = (int)(((long long)K + kStep - 1) / kStep);
  d.KG = (d.KS + 3) / 4;
  return d;
}

// ------------------------------------------------------------- bf16 bits
// fp32 -> bf16, round to nearest even (finite inputs).
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Largest |bf16| of the 8 values in v, as a bf16 magnitude bit pattern.
// Magnitude bit patterns of finite values order like the values themselves,
// so packed 16-bit integer maxima do the work two values at a time.
// mag_mask = 0 treats the 8 values as zeros.
__device__ inline uint32_t amax8_bits(uint4 v, uint32_t mag_mask = 0x7FFF7FFFu) {
  const u16x2 a = __builtin_bit_cast(u16x2, v.x & mag_mask);
  const u16x2 b = __builtin_bit_cast(u16x2, v.y & mag_mask);
  const u16x2 c = __builtin_bit_cast(u16x2, v.z & mag_mask);
  const u16x2 d = __builtin_bit_cast(u16x2, v.w & mag_mask);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Max over the 4 lanes of an aligned quad (lanes 4q..4q+3), by two DPP
// quad permutations.  All four lanes must be active.
__device__ inline uint32_t quad_max(uint32_t x) {
  uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
  x = max(x, y);
  y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
  return max(x, y);
}

// e8m0 scale byte from the group maximum (bf16 magnitude bits): add 2^21 to
// the fp32 pattern (round the maximum up to a power of two when its
// significand is at least 1.75), take the biased exponent e; the unbiased
// scale exponent is e - 127 - 2, clamped to [-127, 127]; the byte is that
// plus 127, i.e. max(e - 2, 0).  (Rule of submission 752099 `_bf16_to_fp4_hw`.)
// On the bf16 pattern the same steps read: add 2^5, exponent = bits 7..14.
__device__ inline uint32_t scale_byte_from_amax(uint32_t amax_bf16_bits) {
  uint32_t e = ((amax_bf16_bits + 0x20u) >> 7) & 0xFFu;
  return e > 2u ? e - 2u : 0u;
}

// Encode 8 bf16 values (v, in memory order) under one scale byte into 8
// e2m1 codes, element i in nibble i of the result (byte j holds elements 2j
// and 2j+1, even element in the low nibble).
//
// gfx950's scaled convert divides each value by the fp32 scale 2^(byte-127)
// (passed as the bit pattern byte << 23), rounds to nearest e2m1 with ties
// to even, saturates at 6 and keeps the sign of zero results -- the element
// rule of submission 694791 `_mxfp4_quant_tile`.  Its results were checked
// against that rule for every finite bf16 value under every scale byte
// 0..253 (byte 0 included, whose pattern reads as +0.0), and the quantizer
// tests repeat that sweep through the library against the CPU oracle.
__device__ inline uint32_t encode8(uint4 v, uint32_t byte) {
  const float scale = __uint_as_float(byte << 23);
  // each convert writes one byte of r (selector 0..3), so all four bytes are
  // written and the starting value (here v.x's register) never shows
  uint32_t r = v.x;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, v.x), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, v.y), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, v.z), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, v.w), scale, 3);
  return r;
}

// ------------------------------------------------- buffer copies to LDS
// Raw buffer access: descriptor word 3 for untyped dword access on CDNA3/4;
// reads past num_records return zero.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;

__device__ inline BufRsrc make_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, kBufWord3);
}
// Asynchronous copy global -> LDS: lane L's 16 (or 4) bytes at voff + soff
// land at lds + 16 L (or 4 L); lds is wave-uniform.
typedef __attribute__((address_space(3))) void* LdsPtr;
constexpr int kCachePolicyNT = 2;  // cache-policy operand of buffer loads: nontemporal
__device__ inline void dma16(BufRsrc r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 16, voff, soff, 0, 0);
}
__device__ inline void dma4(BufRsrc r, uint8_t* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LdsPtr)lds, 4, voff, soff, 0, 0);
}

// ------------------------------------------------------ matrix instruction
// One gfx950 block-scaled 16x16x128 FP4 x FP4 product-accumulate.
//   a: this lane's 32 A codes (row L%16, K-group L/16), 16 bytes;
//   b: this lane's 32 B codes (column L%16, K-group L/16), 16 bytes;
//   sa, sb: this lane's e8m0 scale bytes (low byte used);
//   acc: 4 fp32 of C, rows 4*(L/16)+e, column L%16.
__device__ inline f32x4 mfma_fp4(uint4 a, uint4 b, f32x4 acc, int sa, int sb) {
  i32x8 a8 = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  i32x8 b8 = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  // format 4 = e2m1 for both operands; byte 0 of each scale register.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, acc, 4, 4, 0, sa, 0, sb);
}

}  // namespace mx
