// Device-side building blocks shared by the Evoformer attention kernels (gfx950 only).
//
// MFMA tile conventions (v_mfma_f32_32x32x16_{f16,bf16}, wave64), measured on
// the device:
//   A operand (32 x 16): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B operand (16 x 32): lane l holds B[8*(l/32) + e][l % 32]
//   C/D       (32 x 32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// so a lane always owns one output column and 16 rows in four runs of four.
//
// ds_read_b64_tr_b16, per group of 16 lanes: lane i supplies the address of
// four consecutive 16-bit elements M[i][0..3]; lane j receives
// M[4*e + j/4][j % 4] for e = 0..3.  Pointing lane i at
// &X[k0 + i/4][n0 + 4*(i%4)] of a row-major X therefore hands lane j the
// column X[k0..k0+3][n0 + j]: the transposed operand fetch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- dtypes

struct F16 {
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  // two floats -> packed pair (round to nearest even)
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ floatx16 mfma(const short8_t& a, const short8_t& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  // mixed fma: a*b + (float)h, h a stored 16-bit value
  static __device__ __forceinline__ float fma_mix(float a, float b, uint16_t h) {
    return __builtin_fmaf(a, b, (float)__builtin_bit_cast(_Float16, h));
  }
};

struct BF16 {
  static __device__ __forceinline__ float to_f32(uint16_t b) {
    return __builtin_bit_cast(float, ((uint32_t)b) << 16);
  }
  static __device__ __forceinline__ uint16_t from_f32(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ floatx16 mfma(const short8_t& a, const short8_t& b, const floatx16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float fma_mix(float a, float b, uint16_t h) {
    return __builtin_fmaf(a, b, to_f32(h));
  }
};

// ------------------------------------------------------------ lane helpers

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap).
// Written as inline assembly: the compiler's model of the builtin with both
// operands equal drops the swapped copy, so it is not used here.  The s_nop
// pads cover the VALU-write -> permlane-read hazard on either side.
__device__ __forceinline__ void xhalf_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xhalf_max(float x) {
  float a = x, b = x;
  xhalf_swap(a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float xhalf_sum(float x) {
  float a = x, b = x;
  xhalf_swap(a, b);
  return a + b;
}

// Transposed 4x16-bit fetch from LDS (see the header comment).
__device__ __forceinline__ short4_t lds_read_tr(const uint16_t* lds_base, int elem_offset) {
  const lds_u16* p = (const lds_u16*)(lds_base) + elem_offset;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

__device__ __forceinline__ short8_t cat4(short4_t a, short4_t b) {
  short8_t r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return r;
}

// Row stride (in 16-bit elements) for an LDS tile whose rows are read 16 bytes
// per lane, one row per lane: a multiple of 4 dwords with an odd multiplier,
// so 16 consecutive rows land on distinct bank quads.
__host__ __device__ constexpr int padded_stride_elems(int min_elems) {
  int dw = (min_elems + 1) / 2;         // dwords needed
  int q = (dw + 3) / 4;                 // quads of dwords
  if ((q & 1) == 0) q += 1;             // odd number of quads
  return q * 8;                         // back to 16-bit elements
}

}  // namespace evo
