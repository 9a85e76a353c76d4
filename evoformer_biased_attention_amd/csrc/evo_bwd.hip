// Recompute-based backward of Evoformer biased attention on gfx950.
//
// DeepSpeed4Science guide §3.7: the backward starts from the saved O and fp32
// lse, derives delta, then the gradients of Q, K, V and of both biases, the
// bias gradients accumulated in fp32 and cast back to the input dtype.
//
//   P   = exp(S - lse)               (S recomputed, never stored)
//   dP  = dO V^T,  delta = rowsum(dO * O)
//   dS  = P * (dP - delta)
//   dV  = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K
//   dmask[b,n,j] = sum_h sum_i dS,  dpair[b,h,i,j] = sum_n dS
//
// The reductions pull in different directions (dK, dV over queries; dQ over
// keys; dpair over n; dmask over heads and queries), so the work is split
// over two kernels that each recompute P, plus one reduction kernel.  Rows
// that fit one key tile use bwd_q3 and bwd_kv3 (evo_bwd_tile.hip).  Longer
// rows use bwd_q3 with one key tile per workgroup (dQ as fp32 partials) and
// the key-side kernel of this file:
//   bwd_kv   a workgroup owns 128 keys of one (b, n, h) (32 per wave) and
//            walks all queries: dK, dV and per-head dmask partials stay in
//            registers.  Operands: S = Q K^T with a lane per key.
//   bwd_fin  dmask = sum_h partials, dpair = sum_g partials, dQ = sum of the
//            key-tile partials, each in a fixed order (bitwise
//            reproducible), then rounded to dtype.
#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

template <int D, bool HAS_MASK>
struct BwdShape {
  static constexpr int KSTEPS_D = (D + 15) / 16;
  static constexpr bool AUG_IN_PAD = (D % 16) != 0;
  static constexpr int KSTEPS = KSTEPS_D + ((HAS_MASK && !AUG_IN_PAD) ? 1 : 0);
  static constexpr int KW = KSTEPS * 16;               // Q'/K' row width incl. mask columns
  static constexpr int KS = padded_stride_elems(KW > 32 ? KW : 32);  // row-read + tr-read tile
  static constexpr int VW = D < 32 ? 32 : D;
  static constexpr int DS = padded_stride_elems(VW);   // dO / V tile stride
  static constexpr int MB = (D + 31) / 32;
  static constexpr int RW = KSTEPS_D * 16;             // columns read row-wise (zero beyond D)
};

// 8 values of row `row` starting at column c of a [.., D] tensor, with the
// mask-augmentation pattern beyond D: Q side {s_hi, s_lo}, K side {m, m'}.
template <int D>
__device__ __forceinline__ short8_t load_row8(const uint16_t* row, int c, bool valid, bool has_mask, uint16_t aug0,
                                              uint16_t aug1) {
  short8_t r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c + 8 <= D) {
    if (valid) r = *reinterpret_cast<const short8_t*>(row + c);
  } else if (has_mask) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int a = c + e - D;
      r[e] = (short)(a == 0 ? aug0 : (a == 1 ? aug1 : 0));
    }
  }
  return r;
}

__device__ __forceinline__ uint16_t pick16b(const u32x2 (&b)[4], int r) {
  uint32_t w = b[r / 4][(r % 4) / 2];
  return (r & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
}

// ----------------------------------------------------------------- bwd_kv

constexpr int kKvWaves = 4;
constexpr int kKvKeys = 32 * kKvWaves;

template <class T, int D, bool HAS_MASK, bool HAS_PAIR, bool WANT_DMASK>
__global__ __launch_bounds__(256, 2) void evo_bwd_kv_kernel(BwdArgs a) {
  using S = BwdShape<D, HAS_MASK>;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[32 * S::KS];     // Q' rows of the query block (with {s_hi, s_lo})
  __shared__ __attribute__((aligned(16))) uint16_t sdO[32 * S::DS];    // dO rows of the query block
  __shared__ __attribute__((aligned(16))) uint16_t sB2[HAS_PAIR ? 32 * (kKvKeys + 32) : 1];  // pair[i][j-tile]
  __shared__ __attribute__((aligned(16))) float sNL[32];               // -lse*log2e (0 -> p = 0 rows use +inf lse)
  __shared__ __attribute__((aligned(16))) float sDel[32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int L = a.L, H = a.H, N = a.N;
  const int jtiles = (L + kKvKeys - 1) / kKvKeys;
  // h fastest, then key tile, then n: one XCD covers whole rows of a run of slices
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int jt = rest % jtiles;
  rest /= jtiles;
  const int n = rest % N;
  const int b = rest / N;
  const size_t slice = ((size_t)b * N + n) * L;
  const int j = jt * kKvKeys + wave * 32 + (lane & 31);
  const bool j_valid = j < L;
  constexpr int B2S = kKvKeys + 32;  // 80 dwords: 4 rows hit disjoint bank octets

  // ---- stationary K' and V^T operands (B of S = Q' K'^T and dP = dO V^T)
  short8_t kop[S::KSTEPS], vop[S::KSTEPS_D];
  {
    const uint16_t* krow = a.k + ((slice + (j_valid ? j : 0)) * H + h) * D;
    const uint16_t* vrow = a.v + ((slice + (j_valid ? j : 0)) * H + h) * D;
    uint16_t m = 0;
    if constexpr (HAS_MASK) m = j_valid ? a.mask[((size_t)b * N + n) * L + j] : (uint16_t)0;
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s)
      kop[s] = load_row8<D>(krow, 16 * s + 8 * half, j_valid, HAS_MASK, m, a.s_lo != 0 ? m : (uint16_t)0);
#pragma unroll
    for (int s = 0; s < S::KSTEPS_D; ++s) vop[s] = load_row8<D>(vrow, 16 * s + 8 * half, j_valid, false, 0, 0);
  }
  floatx16 dk[S::MB], dv[S::MB];
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) {
    dk[mb] = floatx16{};
    dv[mb] = floatx16{};
  }
  float dmask_acc = 0.f;

  const int nib = (L + 31) / 32;
  for (int ib = 0; ib < nib; ++ib) {
    const int i0 = ib * 32;
    __syncthreads();
    // ---- stage the query block: Q', dO, -lse*log2e, delta, pair tile
    for (int t = tid; t < 32 * (S::KW / 8); t += 256) {
      int r = t / (S::KW / 8), c8 = t % (S::KW / 8);
      int i = i0 + r;
      const uint16_t* qrow = a.q + ((slice + (i < L ? i : 0)) * H + h) * D;
      *reinterpret_cast<short8_t*>(&sQ[r * S::KS + c8 * 8]) =
          load_row8<D>(qrow, c8 * 8, i < L, HAS_MASK, a.s_hi, a.s_lo);
    }
    for (int t = tid; t < 32 * (S::RW / 8); t += 256) {
      int r = t / (S::RW / 8), c8 = t % (S::RW / 8);
      int i = i0 + r;
      short8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (i < L && c8 * 8 < D) v = *reinterpret_cast<const short8_t*>(a.dout + ((slice + i) * H + h) * D + c8 * 8);
      *reinterpret_cast<short8_t*>(&sdO[r * S::DS + c8 * 8]) = v;
    }
    if (tid < 32) {
      int i = i0 + tid;
      float lse = (i < L) ? a.lse[(((size_t)b * N + n) * H + h) * L + i] : kNegInf;
      // rows with lse = -inf (no finite score) get p = 0
      sNL[tid] = (lse == kNegInf) ? kNegInf : -lse * kLog2e;
      sDel[tid] = (i < L) ? a.delta[(((size_t)b * N + n) * H + h) * L + i] : 0.f;
    }
    if constexpr (HAS_PAIR) {
      const bool vec = (L % 8) == 0;
      for (int t = tid; t < 32 * (kKvKeys / 8); t += 256) {
        int r = t / (kKvKeys / 8), c8 = t % (kKvKeys / 8);
        int i = i0 + r, jj = jt * kKvKeys + c8 * 8;
        short8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (i < L) {
          const uint16_t* p = a.pair + (((size_t)b * H + h) * L + i) * L + jj;
          if (vec && jj + 8 <= L) {
            v = *reinterpret_cast<const short8_t*>(p);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (jj + e < L) ? (short)p[e] : (short)0;
          }
        }
        *reinterpret_cast<short8_t*>(&sB2[r * B2S + c8 * 8]) = v;
      }
    }
    __syncthreads();

    // ---- S = Q' K'^T (lane = key j, rows = queries)
    floatx16 acc = floatx16{};
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      short8_t qa = *reinterpret_cast<const short8_t*>(&sQ[(lane & 31) * S::KS + 16 * s + 8 * half]);
      acc = T::mfma(qa, kop[s], acc);
    }
    floatx16 dp = floatx16{};
#pragma unroll
    for (int s = 0; s < S::KSTEPS_D; ++s) {
      short8_t oa = *reinterpret_cast<const short8_t*>(&sdO[(lane & 31) * S::DS + 16 * s + 8 * half]);
      dp = T::mfma(oa, vop[s], dp);
    }
    // rows held: i = 8*(r/4) + 4*half + r%4
    float nl[16], del[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      floatx4 x = *reinterpret_cast<const floatx4*>(&sNL[8 * q + 4 * half]);
      floatx4 y = *reinterpret_cast<const floatx4*>(&sDel[8 * q + 4 * half]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        nl[4 * q + u] = x[u];
        del[4 * q + u] = y[u];
      }
    }
    float sv[16];
    if constexpr (HAS_PAIR) {
      u32x2 pb[4];
      const int qg = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = 8 * q + 4 * half;
        const int n0 = wave * 32 + 16 * (qg & 1);
        short4_t v = lds_read_tr(sB2, (k0 + (i16 >> 2)) * B2S + n0 + 4 * (i16 & 3));
        pb[q] = __builtin_bit_cast(u32x2, v);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = T::fma_mix(acc[r], a.scale, pick16b(pb, r));
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = acc[r] * a.scale;
    }
    uint32_t ppk[8], dspk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = (nl[r] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], kLog2e, nl[r]));
      float p1 = (nl[r + 1] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r + 1], kLog2e, nl[r + 1]));
      float d0 = p0 * (dp[r] - del[r]);
      float d1 = p1 * (dp[r + 1] - del[r + 1]);
      if constexpr (WANT_DMASK) dmask_acc += d0 + d1;
      ppk[r / 2] = T::pack2(p0, p1);
      dspk[r / 2] = T::pack2(d0, d1);
    }
    // ---- dV^T += dO^T P, dK^T += Q^T dS   (k = query, permuted as held)
    const int qg = lane >> 4, i16 = lane & 15, g = qg >> 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      short8_t pb = __builtin_bit_cast(short8_t, u32x4{ppk[4 * t], ppk[4 * t + 1], ppk[4 * t + 2], ppk[4 * t + 3]});
      short8_t db = __builtin_bit_cast(short8_t, u32x4{dspk[4 * t], dspk[4 * t + 1], dspk[4 * t + 2], dspk[4 * t + 3]});
      const int k0 = 16 * t + 4 * g;
#pragma unroll
      for (int mb = 0; mb < S::MB; ++mb) {
        const int n0 = 16 * (qg & 1) + 32 * mb;
        const int r0 = k0 + (i16 >> 2), c0 = n0 + 4 * (i16 & 3);
        short8_t oa = cat4(lds_read_tr(sdO, r0 * S::DS + c0), lds_read_tr(sdO, (r0 + 8) * S::DS + c0));
        dv[mb] = T::mfma(oa, pb, dv[mb]);
        short8_t qa = cat4(lds_read_tr(sQ, r0 * S::KS + c0), lds_read_tr(sQ, (r0 + 8) * S::KS + c0));
        dk[mb] = T::mfma(qa, db, dk[mb]);
      }
    }
  }

  // ---- epilogue: dK = scale * dK^T, dV; per-head dmask partial
  if (j_valid) {
    uint16_t* dkrow = a.dk + ((slice + j) * H + h) * D;
    uint16_t* dvrow = a.dv + ((slice + j) * H + h) * D;
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 32 * mb + 8 * q + 4 * half;
        if (d < D) {
          u32x2 wk, wv;
          wk[0] = T::pack2(dk[mb][4 * q] * a.scale, dk[mb][4 * q + 1] * a.scale);
          wk[1] = T::pack2(dk[mb][4 * q + 2] * a.scale, dk[mb][4 * q + 3] * a.scale);
          wv[0] = T::pack2(dv[mb][4 * q], dv[mb][4 * q + 1]);
          wv[1] = T::pack2(dv[mb][4 * q + 2], dv[mb][4 * q + 3]);
          *reinterpret_cast<u32x2*>(dkrow + d) = wk;
          *reinterpret_cast<u32x2*>(dvrow + d) = wv;
        }
      }
  }
  if constexpr (WANT_DMASK) {
    const float tot = xhalf_sum(dmask_acc);
    if (j_valid && half == 0) a.dmask_part[(((size_t)b * N + n) * H + h) * L + j] = tot;
  }
}

// ---------------------------------------------------------------- bwd_fin

// Reductions in one launch, each in a fixed order (bitwise reproducible):
//   threads [0, n_pair)                  dpair = sum of the n-group partials
//                                        (4 consecutive elements each when
//                                        the count allows 16-byte access);
//   [n_pair, n_pair + n_mask)            dmask = sum of the per-head partials;
//   [n_pair + n_mask, ... + n_dq)        dQ = sum of the key-tile partials
//                                        (rows longer than one key tile), 4
//                                        consecutive elements each.
template <class T, bool VEC>
__global__ __launch_bounds__(256) void evo_bwd_fin_kernel(BwdArgs a, int ngroups, int64_t n_pair, int64_t n_mask,
                                                          int64_t n_dq, int jtiles) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n_pair) {
    const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
    if constexpr (VEC) {
      const int64_t idx = 4 * e;
      floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
      int gg = 0;
      for (; gg + 1 < ngroups; gg += 2) {
        s0 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)gg * per + idx);
        s1 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)(gg + 1) * per + idx);
      }
      if (gg < ngroups) s0 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)gg * per + idx);
      const floatx4 s = s0 + s1;
      *reinterpret_cast<floatx4*>(a.dpair_f32 + idx) = s;
      u32x2 w;
      w[0] = T::pack2(s[0], s[1]);
      w[1] = T::pack2(s[2], s[3]);
      *reinterpret_cast<u32x2*>(a.dpair + idx) = w;
    } else {
      float s0 = 0.f, s1 = 0.f;
      int gg = 0;
      for (; gg + 1 < ngroups; gg += 2) {
        s0 += a.dpair_part[(int64_t)gg * per + e];
        s1 += a.dpair_part[(int64_t)(gg + 1) * per + e];
      }
      if (gg < ngroups) s0 += a.dpair_part[(int64_t)gg * per + e];
      const float s = s0 + s1;
      a.dpair_f32[e] = s;
      a.dpair[e] = T::from_f32(s);
    }
    return;
  }
  const int64_t m = e - n_pair;
  if (m < n_mask) {
    const int j = (int)(m % a.L);
    const int64_t bn = m / a.L;
    float s = 0.f;
    for (int hh = 0; hh < a.H; ++hh) s += a.dmask_part[(bn * a.H + hh) * a.L + j];
    a.dmask_f32[m] = s;
    a.dmask[m] = T::from_f32(s);
    return;
  }
  const int64_t q = m - n_mask;
  if (q < n_dq) {
    const int64_t per = n_dq * 4, idx = 4 * q;
    floatx4 s = *reinterpret_cast<const floatx4*>(a.dq_part + idx);
    for (int jt = 1; jt < jtiles; ++jt) s += *reinterpret_cast<const floatx4*>(a.dq_part + (int64_t)jt * per + idx);
    u32x2 w;
    w[0] = T::pack2(s[0], s[1]);
    w[1] = T::pack2(s[2], s[3]);
    *reinterpret_cast<u32x2*>(a.dq + idx) = w;
  }
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HM, bool HP>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const bool want_dmask = a.dmask != nullptr;
  const bool want_dpair = a.dpair != nullptr;
  const bool fits = a.L <= KVTile<D>::CH;
  const int jtiles = (a.L + KVTile<D>::CH - 1) / KVTile<D>::CH;
  if (fits) {
    const hipError_t e = launch_bwd_tile(a, D, std::is_same<T, BF16>::value, st);
    if (e != hipSuccess) return e;
  } else {
    // bwd_q3 over key tiles (dQ partials, delta, dpair partials), then the
    // key-side kernel, which reads delta
    hipError_t e = launch_bwd_q_split(a, D, std::is_same<T, BF16>::value, st);
    if (e != hipSuccess) return e;
    const int grid = a.B * a.N * a.H * ((a.L + kKvKeys - 1) / kKvKeys);
    prof_begin(K_BWD_KV, st);
    if (want_dmask)
      hipLaunchKernelGGL((evo_bwd_kv_kernel<T, D, HM, HP, true>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((evo_bwd_kv_kernel<T, D, HM, HP, false>), dim3(grid), dim3(256), 0, st, a);
    prof_end(K_BWD_KV, st);
  }
  const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
  const bool vec = (per % 4) == 0;
  const int64_t n_pair = want_dpair ? (vec ? per / 4 : per) : 0;
  const int64_t n_mask = want_dmask ? (int64_t)a.B * a.N * a.L : 0;
  const int64_t n_dq = fits ? 0 : (int64_t)a.B * a.N * a.L * a.H * D / 4;
  if (n_pair + n_mask + n_dq > 0) {
    const unsigned blocks = (unsigned)((n_pair + n_mask + n_dq + 255) / 256);
    prof_begin(K_BWD_FIN, st);
    if (vec)
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, true>), dim3(blocks), dim3(256), 0, st, a, a.n_groups_q, n_pair,
                         n_mask, n_dq, jtiles);
    else
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, false>), dim3(blocks), dim3(256), 0, st, a, a.n_groups_q, n_pair,
                         n_mask, n_dq, jtiles);
    prof_end(K_BWD_FIN, st);
  }
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  const bool hm = a.mask != nullptr, hp = a.pair != nullptr;
  if (hm && hp) return launch_bwd_t<T, D, true, true>(a, s);
  if (hm) return launch_bwd_t<T, D, true, false>(a, s);
  if (hp) return launch_bwd_t<T, D, false, true>(a, s);
  return launch_bwd_t<T, D, false, false>(a, s);
}

template <class T>
static hipError_t launch_bwd_dt(const BwdArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 8: return launch_bwd_d<T, 8>(a, s);
    case 16: return launch_bwd_d<T, 16>(a, s);
    case 32: return launch_bwd_d<T, 32>(a, s);
    case 64: return launch_bwd_d<T, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(BwdArgs a, int D, bool bf16, hipStream_t stream) {
  return bf16 ? launch_bwd_dt<BF16>(a, D, stream) : launch_bwd_dt<F16>(a, D, stream);
}

}  // namespace evo
