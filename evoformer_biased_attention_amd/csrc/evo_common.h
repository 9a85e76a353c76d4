// Device-side building blocks shared by the Evoformer attention kernels (gfx950 only).
//
// MFMA tile conventions (v_mfma_f32_32x32x16_{f16,bf16}, wave64), measured on
// the device:
//   A operand (32 x 16): lane l holds A[l % 32][8*(l/32) + e], e = 0..7
//   B operand (16 x 32): lane l holds B[8*(l/32) + e][l % 32]
//   C/D       (32 x 32): lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// so a lane always owns one output column and 16 rows in four runs of four.
// v_mfma_f32_16x16x32_{f16,bf16}:
//   A (16 x 32): lane l holds A[l % 16][8*(l/16) + e]
//   B (32 x 16): lane l holds B[8*(l/16) + e][l % 16]
//   C (16 x 16): lane l, register r holds C[4*(l/16) + r][l % 16]
//
// ds_read_b64_tr_b16, per group of 16 lanes: lane i supplies the address of
// four consecutive 16-bit elements M[i][0..3]; lane j receives
// M[4*e + j/4][j % 4] for e = 0..3.  Pointing lane i at
// &X[k0 + i/4][n0 + 4*(i%4)] of a row-major X therefore hands lane j the
// column X[k0..k0+3][n0 + j]: the transposed operand fetch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
  static __device__ __forceinline__ floatx4 mfma16(const short8_t& a, const short8_t& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  // v_mfma_f32_16x16x16_f16 (same issue cost as 16x16x32 on gfx950, half the k)
  static __device__ __forceinline__ floatx4 mfma16k16(const short4_t& a, const short4_t& b, const floatx4& c) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4, a), __builtin_bit_cast(h4, b), c, 0, 0, 0);
  }
  // c + a.lo*b.lo + a.hi*b.hi for packed pairs, fp32 accumulation
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
  }
  static __device__ __forceinline__ short one() { return (short)0x3c00; }
  static constexpr uint16_t kNegInfBits = 0xfc00;
  // mixed fma: a*b + (float)h, h a stored 16-bit value
  static __device__ __forceinline__ float fma_mix(float a, float b, uint16_t h) {
    return __builtin_fmaf(a, b, (float)__builtin_bit_cast(_Float16, h));
  }
  // a*b + half of a packed pair, in one v_fma_mix_f32 (the compiler does not
  // form it from a packed register on its own)
  static __device__ __forceinline__ float fma_mix_lo(float a, float b, uint32_t w) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,0,1]" : "=v"(r) : "v"(a), "v"(b), "v"(w));
    return r;
  }
  static __device__ __forceinline__ float fma_mix_hi(float a, float b, uint32_t w) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,1] op_sel_hi:[0,0,1]" : "=v"(r) : "v"(a), "v"(b), "v"(w));
    return r;
  }
  // running row sum of the probabilities: fp16 sums the rounded pair in one
  // v_dot2_f32_f16 (fp32 accumulation; the rounding is 2^-11 relative)
  static __device__ __forceinline__ float rowsum_add(float acc, float, float, uint32_t packed) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, packed), one, acc, false);
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
  static __device__ __forceinline__ floatx4 mfma16(const short8_t& a, const short8_t& b, const floatx4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mfma16k16(const short4_t& a, const short4_t& b, const floatx4& c) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(b4, a), __builtin_bit_cast(b4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
  }
  static __device__ __forceinline__ short one() { return (short)0x3f80; }
  static constexpr uint16_t kNegInfBits = 0xff80;
  static __device__ __forceinline__ float fma_mix(float a, float b, uint16_t h) {
    return __builtin_fmaf(a, b, to_f32(h));
  }
  static __device__ __forceinline__ float fma_mix_lo(float a, float b, uint32_t w) {
    return __builtin_fmaf(a, b, __builtin_bit_cast(float, w << 16));
  }
  static __device__ __forceinline__ float fma_mix_hi(float a, float b, uint32_t w) {
    return __builtin_fmaf(a, b, __builtin_bit_cast(float, w & 0xffff0000u));
  }
  // bf16 rounding (2^-8) is too coarse for the lse: sum the fp32 values
  static __device__ __forceinline__ float rowsum_add(float acc, float p0, float p1, uint32_t) {
    return acc + (p0 + p1);
  }
};

// ------------------------------------------------------------ bias by MFMA
// bf16 has no mixed-precision FMA, so a VALU pair-bias add would widen each
// value first; the bf16 forward and query-side backward add the bias inside
// the score MFMA chain instead,
// with an A operand that holds sqrt(D) on the diagonal of the block's keys
// (the scores' accumulator holds sqrt(D) times each bias, as for the mask).
// sqrt(D) is exact in 16 bits at D = 16 and 64; at D = 8 and 32 it is taken as
// the dtype's rounding plus the rounding of the remainder, two products whose
// sum is within 3e-7 relative (one value alone is off by 1.1e-4).  The
// products are exact in fp32.
template <int D>
constexpr int kSqrtParts = (D == 16 || D == 64) ? 1 : 2;

template <class T>
__device__ __forceinline__ void sqrt_d_parts(float sqrt_d, uint16_t (&p)[2]) {
  p[0] = T::from_f32(sqrt_d);
  p[1] = T::from_f32(sqrt_d - T::to_f32(p[0]));
}

// Wait states between an MFMA result and its use as the accumulator input of an
// MFMA of another opcode (a 16x16x32 score chain into the 16x16x16 bias
// product, both 4 passes).  The compiler inserts none when the accumulator
// registers overlap exactly, as it may between two MFMAs of one opcode, but
// across the two opcodes the result is not reliably there yet.  Measured on
// gfx950: with no wait states the backward's outputs changed from call to call
// on identical inputs; with 4, 6, 8 or 16 every call gave the same bits, equal
// across the four.  6 are used (the passes plus two).  The asm takes the
// accumulator as an operand, so the compiler cannot move either product past it.
__device__ __forceinline__ void mfma_acc_handoff(floatx4& acc) {
  asm volatile("s_nop 5" : "+v"(acc));
}

// bf16 pair-bias bits for such a product: -inf (and the NaNs of negative sign)
// become the most negative finite value, whose product with sqrt(D) still
// overflows to -inf in fp32 while the zeros off the diagonal give 0, not
// 0 * inf = NaN.  One packed 16-bit minimum per two values.
__device__ __forceinline__ uint32_t bf16x2_no_neg_inf(uint32_t w) {
  using u16x2 = unsigned short __attribute__((ext_vector_type(2)));
  const u16x2 lim = {(unsigned short)0xFF7F, (unsigned short)0xFF7F};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, w), lim));
}

// ------------------------------------------------------------ lane helpers

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Combine a value with the one held by lane l ^ 32 (v_permlane32_swap).
// Written as inline assembly: the compiler's model of the builtin with both
// operands equal drops the swapped copy, so it is not used here.  The s_nop
// pads cover the VALU-write -> permlane-read hazard on either side.
__device__ __forceinline__ void xhalf_swap(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
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

// ------------------------------------------------------- K/V tiles in LDS
//
// A tile holds CH keys of one (b, n, h): K rows of D elements, then V rows
// padded to at least 32 elements (the transposed reads of V^T touch 32
// columns; the padding is never used).  Both are filled by
// global_load_lds_dwordx4, which writes 64 consecutive 16-byte chunks per wave
// instruction, so the layout is a dense array of 16-byte chunks.  Chunk c of
// row r sits at position c ^ swz(r).  The swizzle is constant on aligned
// groups of four rows (the transposed reads take a 4 x 4 block of 8-byte
// pieces from four consecutive rows) and has a period of 16 rows (operand
// blocks of 16 rows sit at fixed offsets from a lane's base address).  For
// 64-byte rows it is -(r / 4) mod 4: measured with the 16-row operand reads of
// the 16x16x32 MFMAs, the 32-row reads of the 32x32x16 MFMAs and both
// transposed-read patterns, it runs every one of them at the contiguous-read
// rate, where r / 4 mod 4 left the 16-row b128 reads at about 60 % of it.
template <int C>
__device__ __forceinline__ int kv_swz(int r) {
  if constexpr (C == 4) {
    return (4 - ((r >> 2) & 3)) & 3;
  } else {
    constexpr int R = 16 / C;  // rows per 64-dword bank cycle
    return (r / R) % C;
  }
}

template <int D>
struct KVTile {
  static constexpr int CH = (D == 64) ? 128 : 256;  // keys per tile
  static constexpr int KC = D / 8;                  // 16-byte chunks per K row
  static constexpr int VC = (D < 32 ? 32 : D) / 8;  // 16-byte chunks per V row
  static constexpr int KCH = CH * KC;
  static constexpr int VCH = CH * VC;
  static constexpr int TCH = KCH + VCH;             // chunks per tile (a multiple of 256)
  static constexpr int BUF_BYTES = TCH * 16;
  static_assert(TCH % 256 == 0, "tile must split evenly over 256 threads");
};

// byte offset of element (row, col) in a swizzled tile with C chunks per row
template <int C>
__device__ __forceinline__ int tr_off(int row, int col) {
  return (row * C + ((col >> 3) ^ kv_swz<C>(row))) * 16 + (col & 7) * 2;
}

__device__ __forceinline__ short4_t lds_read_tr_b(const uint8_t* base, int byte_off) {
  const __attribute__((address_space(3))) uint8_t* p = (const __attribute__((address_space(3))) uint8_t*)base + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
}

// The same transposed read as inline assembly.  The compiler treats the
// builtin as possibly aliasing every LDS copy still in flight from
// global_load_lds and waits for all of them (vmcnt(0)) before it, which
// would stall on the next tile's prefetch.  Reads issued this way are not
// tracked by the compiler: call lds_wait() before using their results.
// Buffers being filled by global_load_lds are never read this way before the
// s_waitcnt + barrier that completes them.
__device__ __forceinline__ short4_t lds_read_tr_asm(const uint8_t* base, int byte_off) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const uint32_t addr = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)base + byte_off);
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return __builtin_bit_cast(short4_t, r);
}
// A 16-byte LDS read in the same style (not tracked by the compiler).
__device__ __forceinline__ short8_t lds_read_b128_asm(const uint8_t* base, int byte_off) {
  const uint32_t addr = (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)base + byte_off);
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return __builtin_bit_cast(short8_t, r);
}

// Wait for the reads above and make the waited registers outputs of the wait,
// so that no consumer can be scheduled before it.
__device__ __forceinline__ void lds_wait(short4_t& a, short4_t& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)::"memory");
}
__device__ __forceinline__ void lds_wait(short4_t& a, short4_t& b, short4_t& c, short4_t& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d)::"memory");
}
template <int N, int M>
__device__ __forceinline__ void lds_wait_all(short4_t (&r)[N], short8_t (&s)[M]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+v"(r[k]));
#pragma unroll
  for (int k = 0; k < M; ++k) asm volatile("" : "+v"(s[k]));
}
template <int N>
__device__ __forceinline__ void lds_wait_all(short4_t (&r)[N]) {
  static_assert(N % 2 == 0, "pairs");
  if constexpr (N == 2) {
    lds_wait(r[0], r[1]);
  } else if constexpr (N == 4) {
    lds_wait(r[0], r[1], r[2], r[3]);
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < N; ++k) asm volatile("" : "+v"(r[k]));
  }
}

// Wait for every LDS read in flight, placed after the instructions that
// produce `a` (and `b`): they are operands of the wait, so the scheduler
// cannot hoist it above them.  A wait with only a memory clobber may be
// scheduled above plain ALU work, which then stalls on reads issued just
// before it instead of covering their latency.
template <class A>
__device__ __forceinline__ void lgkm_wait_after(A& a) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a)::"memory");
}
template <class A, class B>
__device__ __forceinline__ void lgkm_wait_after(A& a, B& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)::"memory");
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

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(static_cast<F&&>(f));
  }
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Transposed read (as lds_read_tr_asm) at a compile-time byte offset from a
// base address register: the offset goes into the instruction's 16-bit field.
template <int OFF>
__device__ __forceinline__ short4_t lds_tr_imm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return __builtin_bit_cast(short4_t, r);
}

// 16-byte LDS read at a compile-time byte offset, not tracked by the
// compiler (see lds_read_tr_asm): wait with lgkm_wait() and mark the result
// with reg_touch() before using it.
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128_imm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Wait until at most N LDS (and scalar-memory) operations are outstanding.
// LDS reads complete in issue order, so this waits for every LDS read issued
// before the last N of them, whatever scalar loads are also in flight.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).  Issued
// through the builtin so that the compiler's own wait insertion knows what
// has completed; the empty asm statements keep memory accesses on their side.
constexpr unsigned kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr unsigned kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// Wait until every vector memory operation of this thread has completed:
// loads, asynchronous copies into LDS, and stores.
__device__ __forceinline__ void vm_wait_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  asm volatile("" ::: "memory");
}

// Workgroup barrier for LDS: waits for this thread's LDS operations only, not
// for its global stores still in flight (a __syncthreads() also waits for
// those).  Callers complete their asynchronous LDS copies with vm_wait_all()
// before it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Make a register value an output of an (empty) asm placed after a wait, so
// that no use of it is scheduled before the wait.
template <class R>
__device__ __forceinline__ void reg_touch(R& r) {
  asm volatile("" : "+v"(r));
}

}  // namespace evo
