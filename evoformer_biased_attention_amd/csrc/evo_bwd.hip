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
// keys; dpair over n; dmask over heads and queries), so the work is split:
//   bwd_pre  delta = rowsum(dO * O), one thread per row.
//   bwd_kv   a workgroup owns 128 keys of one (b, n, h) (32 per wave) and
//            walks all queries: dK, dV and per-head dmask partials stay in
//            registers.  Operands: S = Q K^T with a lane per key.
//   bwd_q    a workgroup owns 32 queries of one (b, h) and a group of n; its
//            4 waves split the keys.  dQ is summed over the waves in LDS per
//            n; dpair is summed over the n of the group in registers and
//            written once per group as an fp32 partial.  Operands:
//            S^T = K Q^T with a lane per query.
//   bwd_fin  dmask = sum_h partials, dpair = sum_g partials, both in a fixed
//            order (bitwise reproducible), then rounded to dtype.
// Both bwd_kv and bwd_q recompute P from lse; that costs one extra QK^T and
// exp per score but keeps every reduction on chip and free of atomics.
#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

constexpr float kLn2 = 0.6931471805599453f;

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

// ---------------------------------------------------------------- bwd_pre

template <class T, int D>
__global__ __launch_bounds__(256) void evo_bwd_pre_kernel(BwdArgs a) {
  const int64_t rows = (int64_t)a.B * a.N * a.L * a.H;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int h = (int)(r % a.H);
  const int64_t t = r / a.H;
  const int i = (int)(t % a.L);
  const int64_t bn = t / a.L;
  const uint16_t* o = a.out + r * D;
  const uint16_t* g = a.dout + r * D;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    short8_t ov = *reinterpret_cast<const short8_t*>(o + c);
    short8_t gv = *reinterpret_cast<const short8_t*>(g + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf(T::to_f32((uint16_t)ov[e]), T::to_f32((uint16_t)gv[e]), s);
  }
  a.delta[(bn * a.H + h) * a.L + i] = s;
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

// ------------------------------------------------------------------ bwd_q

constexpr int kQWaves = 4;
constexpr int kQChunk = 32 * kQWaves;  // keys staged per step; wave w takes block w

template <class T, int D, bool HAS_MASK, bool HAS_PAIR, bool WANT_DPAIR, int DPC>
__global__ __launch_bounds__(256, 2) void evo_bwd_q_kernel(BwdArgs a) {
  using S = BwdShape<D, HAS_MASK>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kQChunk * S::KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kQChunk * S::DS];
  __shared__ __attribute__((aligned(16))) float sRed[kQWaves * 32 * S::MB * 32];  // dQ^T partials of the 4 waves

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, half = lane >> 5;
  const int L = a.L, H = a.H, N = a.N;
  const int iblocks = (L + 31) / 32;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int ib = rest % iblocks;
  rest /= iblocks;
  const int ng = rest % a.n_groups_q;
  const int b = rest / a.n_groups_q;
  const int i = ib * 32 + (lane & 31);
  const bool i_valid = i < L;
  const int n_begin = ng * a.Gq, n_end = min(N, n_begin + a.Gq);
  const int nchunks = (L + kQChunk - 1) / kQChunk;

  floatx16 dpacc[DPC > 0 ? DPC : 1];
#pragma unroll
  for (int c = 0; c < (DPC > 0 ? DPC : 1); ++c) dpacc[c] = floatx16{};

  const uint16_t* prow = nullptr;
  if constexpr (HAS_PAIR) prow = a.pair + (((size_t)b * H + h) * L + (i_valid ? i : 0)) * L;
  const bool pvec = (L % 4) == 0;

  for (int n = n_begin; n < n_end; ++n) {
    const size_t slice = ((size_t)b * N + n) * L;
    short8_t qop[S::KSTEPS], gop[S::KSTEPS_D];
    {
      const uint16_t* qrow = a.q + ((slice + (i_valid ? i : 0)) * H + h) * D;
      const uint16_t* grow = a.dout + ((slice + (i_valid ? i : 0)) * H + h) * D;
#pragma unroll
      for (int s = 0; s < S::KSTEPS; ++s)
        qop[s] = load_row8<D>(qrow, 16 * s + 8 * half, i_valid, HAS_MASK, a.s_hi, a.s_lo);
#pragma unroll
      for (int s = 0; s < S::KSTEPS_D; ++s) gop[s] = load_row8<D>(grow, 16 * s + 8 * half, i_valid, false, 0, 0);
    }
    float nl = kNegInf, del = 0.f;
    if (i_valid) {
      const size_t ri = (((size_t)b * N + n) * H + h) * L + i;
      float lse = a.lse[ri];
      nl = (lse == kNegInf) ? kNegInf : -lse * kLog2e;
      del = a.delta[ri];
    }
    floatx16 dq[S::MB];
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) dq[mb] = floatx16{};

#pragma unroll
    for (int cu = 0; cu < (DPC > 0 ? DPC : 1); ++cu) {
      for (int c = (DPC > 0 ? cu : 0); c < (DPC > 0 ? cu + 1 : nchunks); ++c) {
        if (c >= nchunks) break;
        const int kc0 = c * kQChunk;
        __syncthreads();
        // ---- stage K' (with mask columns) and V rows of this chunk
        for (int t = tid; t < kQChunk * (S::KW / 8); t += 256) {
          int r = t / (S::KW / 8), c8 = t % (S::KW / 8);
          int jj = kc0 + r;
          const uint16_t* krow = a.k + ((slice + (jj < L ? jj : 0)) * H + h) * D;
          uint16_t m = 0;
          if constexpr (HAS_MASK) m = (jj < L) ? a.mask[((size_t)b * N + n) * L + jj] : (uint16_t)0;
          *reinterpret_cast<short8_t*>(&sK[r * S::KS + c8 * 8]) =
              load_row8<D>(krow, c8 * 8, jj < L, HAS_MASK, m, a.s_lo != 0 ? m : (uint16_t)0);
        }
        for (int t = tid; t < kQChunk * (S::RW / 8); t += 256) {
          int r = t / (S::RW / 8), c8 = t % (S::RW / 8);
          int jj = kc0 + r;
          short8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
          if (jj < L && c8 * 8 < D) v = *reinterpret_cast<const short8_t*>(a.v + ((slice + jj) * H + h) * D + c8 * 8);
          *reinterpret_cast<short8_t*>(&sV[r * S::DS + c8 * 8]) = v;
        }
        __syncthreads();
        const int j0 = kc0 + wave * 32;
        if (j0 < L) {
          // ---- S^T = K' Q'^T and dP^T = V dO^T (lane = query i)
          floatx16 acc = floatx16{}, dp = floatx16{};
#pragma unroll
          for (int s = 0; s < S::KSTEPS; ++s) {
            short8_t ka = *reinterpret_cast<const short8_t*>(&sK[(wave * 32 + (lane & 31)) * S::KS + 16 * s + 8 * half]);
            acc = T::mfma(ka, qop[s], acc);
          }
#pragma unroll
          for (int s = 0; s < S::KSTEPS_D; ++s) {
            short8_t va = *reinterpret_cast<const short8_t*>(&sV[(wave * 32 + (lane & 31)) * S::DS + 16 * s + 8 * half]);
            dp = T::mfma(va, gop[s], dp);
          }
          float sv[16];
          if constexpr (HAS_PAIR) {
            u32x2 pb[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              int jj = j0 + 8 * q + 4 * half;
              u32x2 v = {0u, 0u};
              if (i_valid) {
                if (pvec && jj + 4 <= L) {
                  v = *reinterpret_cast<const u32x2*>(prow + jj);
                } else {
                  uint16_t tt[4];
#pragma unroll
                  for (int u = 0; u < 4; ++u) tt[u] = (jj + u < L) ? prow[jj + u] : (uint16_t)0;
                  v[0] = (uint32_t)tt[0] | ((uint32_t)tt[1] << 16);
                  v[1] = (uint32_t)tt[2] | ((uint32_t)tt[3] << 16);
                }
              }
              pb[q] = v;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = T::fma_mix(acc[r], a.scale, pick16b(pb, r));
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = acc[r] * a.scale;
          }
          uint32_t dspk[8];
          float ds[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int jj = j0 + 8 * (r / 4) + 4 * half + (r % 4);
            float p = (nl == kNegInf || jj >= L) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], kLog2e, nl));
            ds[r] = p * (dp[r] - del);
          }
#pragma unroll
          for (int r = 0; r < 16; r += 2) dspk[r / 2] = T::pack2(ds[r], ds[r + 1]);
          if constexpr (WANT_DPAIR && DPC > 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) dpacc[cu][r] += ds[r];
          } else if constexpr (WANT_DPAIR) {
            // long rows: accumulate straight into the fp32 result (order not fixed)
            if (i_valid) {
              float* dst = a.dpair_f32 + (((size_t)b * H + h) * L + i) * L;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int jj = j0 + 8 * (r / 4) + 4 * half + (r % 4);
                if (jj < L) atomicAdd(dst + jj, ds[r]);
              }
            }
          }
          // ---- dQ^T += K^T dS^T  (A = K^T by transposed reads, k = key as held)
          const int qg = lane >> 4, i16 = lane & 15, g = qg >> 1;
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            short8_t db = __builtin_bit_cast(short8_t, u32x4{dspk[4 * t], dspk[4 * t + 1], dspk[4 * t + 2], dspk[4 * t + 3]});
            const int k0 = wave * 32 + 16 * t + 4 * g;
#pragma unroll
            for (int mb = 0; mb < S::MB; ++mb) {
              const int r0 = k0 + (i16 >> 2), c0 = 16 * (qg & 1) + 32 * mb + 4 * (i16 & 3);
              short8_t ka = cat4(lds_read_tr(sK, r0 * S::KS + c0), lds_read_tr(sK, (r0 + 8) * S::KS + c0));
              dq[mb] = T::mfma(ka, db, dq[mb]);
            }
          }
        }
      }
    }
    // ---- sum the 4 waves' dQ^T partials, write dQ = scale * dQ
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sRed[((wave * S::MB + mb) * 16 + r) * 64 + lane] = dq[mb][r];
    __syncthreads();
    {
      // thread t sums element e = t (+256k) of the 16*MB*64 per-wave values
      constexpr int E = 16 * S::MB * 64;
      for (int e = tid; e < E; e += 256) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kQWaves; ++w) s += sRed[w * E + e];
        const int ln = e % 64, r = (e / 64) % 16, mb = e / (64 * 16);
        const int ii = ib * 32 + (ln & 31);
        const int d = 32 * mb + 8 * (r / 4) + 4 * (ln >> 5) + (r % 4);
        if (ii < L && d < D) a.dq[((slice + ii) * H + h) * D + d] = T::from_f32(s * a.scale);
      }
    }
  }

  if constexpr (WANT_DPAIR && DPC > 0) {
    if (i_valid) {
      float* dst = a.dpair_part + ((((size_t)ng * a.B + b) * H + h) * L + i) * L;
#pragma unroll
      for (int cu = 0; cu < DPC; ++cu) {
        const int j0 = cu * kQChunk + wave * 32;
        if (j0 < L) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int jj = j0 + 8 * q + 4 * half;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (jj + u < L) dst[jj + u] = dpacc[cu][4 * q + u];
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------- bwd_q2
//
// Query-stationary backward for rows that fit one key tile (L <= KVTile::CH),
// on 16x16x32 MFMA tiles so that a wave owns 16 queries:
//   workgroup = 4 waves = 64 queries of one (b, h) and a group of n;
//   per n, K and V of the slice arrive in LDS by asynchronous copies
//   (double-buffered, prefetched one slice ahead), and each wave walks all
//   keys 32 at a time:
//     S^T = K Q^T and dP^T = V dO^T (lane = query, 4 keys per 16-key block),
//     P = exp(S - lse), dS^T = P (dP^T - delta),
//     dQ^T += K^T dS^T (K^T by transposed LDS reads),
//     dpair^T += dS^T, accumulated by an MFMA against a 0/1 selection matrix
//     so that the n-sum costs no VALU work; it stays in registers for the
//     whole n-group and is written once as an fp32 partial.
constexpr int kQ2Rows = 64;

template <class T, int D, bool HAS_MASK, bool HAS_PAIR, bool WANT_DPAIR>
__global__ __launch_bounds__(256, 2) void evo_bwd_q2_kernel(BwdArgs a) {
  using TL = KVTile<D>;
  constexpr int KS32 = (D + 31) / 32;       // 32-wide k-steps over d
  constexpr bool AUG_PAD = (D % 32) != 0;   // D = 8, 16: mask slots follow d in the last step
  constexpr int KSTEPS = KS32 + ((HAS_MASK && !AUG_PAD) ? 1 : 0);
  constexpr int NB = TL::CH / 16;           // 16-key blocks per tile
  constexpr int MB = (D + 15) / 16;         // 16-row blocks of dQ^T
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint16_t smask[2][TL::CH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int L = a.L, H = a.H, N = a.N;
  const int itiles = (L + kQ2Rows - 1) / kQ2Rows;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int it = rest % itiles;
  rest /= itiles;
  const int ng = rest % a.n_groups_q;
  const int b = rest / a.n_groups_q;
  const int i = it * kQ2Rows + wave * 16 + col;
  const bool i_valid = i < L;
  const int ic = min(i, L - 1);
  const int n_begin = ng * a.Gq, n_end = min(N, n_begin + a.Gq);
  const int ntiles = n_end - n_begin;

  // resident pair bias: block blk, lane gets pair[ic][16 blk + 4 g + 0..3]
  u32x2 pbias[HAS_PAIR ? NB : 1];
  if constexpr (HAS_PAIR) {
    const uint16_t* prow = a.pair + (((size_t)b * H + h) * L + ic) * L;
    const bool pvec = (L % 4) == 0;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int j = 16 * blk + 4 * g;
      u32x2 v;
      if (pvec) {
        v = *reinterpret_cast<const u32x2*>(prow + min(j, L - 4));
      } else {
        uint32_t t4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t4[u] = prow[min(j + u, L - 1)];
        v[0] = t4[0] | (t4[1] << 16);
        v[1] = t4[2] | (t4[3] << 16);
      }
      pbias[blk] = v;
    }
  }
  // 0/1 selection operands: slot e of lane group g is key 4g + (e & 3) of block e / 4
  short8_t sel[2];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sel[0][e] = (e < 4 && 4 * g + e == col) ? T::one() : (short)0;
    sel[1][e] = (e >= 4 && 4 * g + (e - 4) == col) ? T::one() : (short)0;
  }
  short8_t qaug = {0, 0, 0, 0, 0, 0, 0, 0};
  if (HAS_MASK && g == 0) {
    qaug[0] = (short)a.s_hi;
    qaug[1] = (short)a.s_lo;
  }

  short8_t qop[KS32], gop[KS32], qnx[KS32], gnx[KS32], onx[KS32];
  float nl = 0.f, del = 0.f, nl_nx = 0.f;
  uint32_t mreg = 0;
  // Q, dO and O rows of this lane's query (8 columns per k-step), and its lse;
  // delta = rowsum(dO * O) is formed from them at the start of the slice
  auto load_rows = [&](int n) {
    const size_t row = (((size_t)b * N + n) * L + ic) * H + h;
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int d0 = 32 * s + 8 * g;
      short8_t qv = {0, 0, 0, 0, 0, 0, 0, 0}, gv = {0, 0, 0, 0, 0, 0, 0, 0}, ov = {0, 0, 0, 0, 0, 0, 0, 0};
      if (d0 + 8 <= D) {
        qv = *reinterpret_cast<const short8_t*>(a.q + row * D + d0);
        gv = *reinterpret_cast<const short8_t*>(a.dout + row * D + d0);
        ov = *reinterpret_cast<const short8_t*>(a.out + row * D + d0);
      } else if (HAS_MASK && AUG_PAD && d0 == D) {
        qv[0] = (short)a.s_hi;
        qv[1] = (short)a.s_lo;
      }
      qnx[s] = qv;
      gnx[s] = gv;
      onx[s] = ov;
    }
    nl_nx = a.lse[(((size_t)b * N + n) * H + h) * L + ic];
  };
  // mask of the tile's keys; keys past L get -inf (HAS_MASK also covers
  // ragged rows without a user mask), so the products themselves mask the tail
  auto load_mask = [&](int n) {
    if constexpr (HAS_MASK) {
      if (tid < TL::CH) mreg = a.mask ? a.mask[((size_t)b * N + n) * L + min(tid, L - 1)] : 0u;
    }
  };
  auto store_mask = [&](int buf) {
    if constexpr (HAS_MASK) {
      if (tid < TL::CH) smask[buf][tid] = (tid < L) ? (uint16_t)mreg : T::kNegInfBits;
    }
  };

  floatx4 dpacc[WANT_DPAIR ? NB : 1];
#pragma unroll
  for (int blk = 0; blk < (WANT_DPAIR ? NB : 1); ++blk) dpacc[blk] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (ntiles > 0) {
    load_mask(n_begin);
    issue_kv_tile<D>(smem, a.k, a.v, ((size_t)b * N + n_begin) * L, 0, L, H, h, wave, lane);
    load_rows(n_begin);
    store_mask(0);
  }
  for (int t = 0; t < ntiles; ++t) {
    const int n = n_begin + t;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      qop[s] = qnx[s];
      gop[s] = gnx[s];
    }
    nl = (nl_nx == kNegInf) ? kNegInf : -nl_nx * kLog2e;  // rows with no finite score: p = 0
    {
      // delta of this lane's query: partial dot over its columns, then the
      // four lane groups holding the same query are summed
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < KS32; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part = __builtin_fmaf(T::to_f32((uint16_t)gnx[s][e]), T::to_f32((uint16_t)onx[s][e]), part);
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      del = part;
      if (g == 0 && i_valid) a.delta[(((size_t)b * N + n) * H + h) * L + i] = del;
    }
    if (t + 1 < ntiles) {
      load_mask(n + 1);
      issue_kv_tile<D>(smem + ((t + 1) & 1) * TL::BUF_BYTES, a.k, a.v, ((size_t)b * N + n + 1) * L, 0, L, H, h, wave,
                       lane);
      load_rows(n + 1);
    }
    const uint8_t* kb = smem + (t & 1) * TL::BUF_BYTES;
    const uint8_t* vb = kb + TL::KCH * 16;
    const uint16_t* mk = smask[t & 1];

    auto kop = [&](int blk, int s) -> short8_t {
      const int r = blk * 16 + col;
      const int c = 4 * s + g;
      short8_t op = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c < TL::KC) {
        op = *reinterpret_cast<const short8_t*>(kb + (r * TL::KC + (c ^ kv_swz<TL::KC>(r))) * 16);
      } else if (HAS_MASK && AUG_PAD && c == TL::KC) {
        const uint16_t m = mk[r];
        op[0] = (short)m;
        op[1] = (short)(a.s_lo != 0 ? m : 0);
      }
      return op;
    };
    auto sblk = [&](int blk) -> floatx4 {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS32; ++s) acc = T::mfma16(kop(blk, s), qop[s], acc);
      if constexpr (HAS_MASK && !AUG_PAD) {
        short8_t op = {0, 0, 0, 0, 0, 0, 0, 0};
        if (g == 0) {
          const uint16_t m = mk[blk * 16 + col];
          op[0] = (short)m;
          op[1] = (short)(a.s_lo != 0 ? m : 0);
        }
        acc = T::mfma16(op, qaug, acc);
      }
      return acc;
    };
    auto dpblk = [&](int blk) -> floatx4 {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const int r = blk * 16 + col;
#pragma unroll
      for (int s = 0; s < KS32; ++s) {
        const int c = 4 * s + g;
        short8_t op = {0, 0, 0, 0, 0, 0, 0, 0};
        if (c < D / 8) op = *reinterpret_cast<const short8_t*>(vb + (r * TL::VC + (c ^ kv_swz<TL::VC>(r))) * 16);
        acc = T::mfma16(op, gop[s], acc);
      }
      return acc;
    };

    floatx4 dq[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dq[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    floatx4 sc[2][2], dp[2][2];
    sc[0][0] = sblk(0);
    sc[0][1] = sblk(1);
    dp[0][0] = dpblk(0);
    dp[0][1] = dpblk(1);
#pragma unroll
    for (int st = 0; st < NB / 2; ++st) {
      if (32 * st < L) {
        const int cur = st & 1;
        // next step's products run under this step's VALU work
        if (st + 1 < NB / 2 && 32 * (st + 1) < L) {
          sc[cur ^ 1][0] = sblk(2 * st + 2);
          sc[cur ^ 1][1] = sblk(2 * st + 3);
          dp[cur ^ 1][0] = dpblk(2 * st + 2);
          dp[cur ^ 1][1] = dpblk(2 * st + 3);
        }
        // K^T operands of dQ^T for this step (transposed reads, waited on below)
        short4_t kt[2 * MB];  // [mb][lo/hi]
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c0 = 16 * mb + 4 * (col & 3);
          const int r0 = 32 * st + 4 * g + (col >> 2);
          kt[2 * mb] = lds_read_tr_asm(kb, tr_off<TL::KC>(r0, c0));
          kt[2 * mb + 1] = lds_read_tr_asm(kb, tr_off<TL::KC>(r0 + 16, c0));
        }
        float ds[2][4];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int blk = 2 * st + hb;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s;
            if constexpr (HAS_PAIR) {
              const uint32_t w = pbias[blk][r / 2];
              s = (r & 1) ? T::fma_mix_hi(sc[cur][hb][r], a.scale, w) : T::fma_mix_lo(sc[cur][hb][r], a.scale, w);
            } else {
              s = sc[cur][hb][r] * a.scale;
            }
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, kLog2e, nl));
            ds[hb][r] = p * (dp[cur][hb][r] - del);
          }
        }
        const short8_t dsb = __builtin_bit_cast(
            short8_t, u32x4{T::pack2(ds[0][0], ds[0][1]), T::pack2(ds[0][2], ds[0][3]), T::pack2(ds[1][0], ds[1][1]),
                            T::pack2(ds[1][2], ds[1][3])});
        if constexpr (WANT_DPAIR) {
          dpacc[2 * st] = T::mfma16(sel[0], dsb, dpacc[2 * st]);
          dpacc[2 * st + 1] = T::mfma16(sel[1], dsb, dpacc[2 * st + 1]);
        }
        lds_wait_all(kt);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dq[mb] = T::mfma16(cat4(kt[2 * mb], kt[2 * mb + 1]), dsb, dq[mb]);
      }
    }
    // ---- dQ = scale * dQ^T: lane holds d = 16 mb + 4 g + 0..3 of query i
    if (i_valid) {
      uint16_t* dqrow = a.dq + ((((size_t)b * N + n) * L + i) * H + h) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int d = 16 * mb + 4 * g;
        if (d < D) {
          u32x2 w;
          w[0] = T::pack2(dq[mb][0] * a.scale, dq[mb][1] * a.scale);
          w[1] = T::pack2(dq[mb][2] * a.scale, dq[mb][3] * a.scale);
          *reinterpret_cast<u32x2*>(dqrow + d) = w;
        }
      }
    }
    if (t + 1 < ntiles) store_mask((t + 1) & 1);
  }

  if constexpr (WANT_DPAIR) {
    if (i_valid) {
      float* dst = a.dpair_part + ((((size_t)ng * a.B + b) * H + h) * L + i) * L;
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int j = 16 * blk + 4 * g;
        if (j + 4 <= L && (L % 4) == 0) {
          *reinterpret_cast<floatx4*>(dst + j) = dpacc[blk];
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (j + u < L) dst[j + u] = dpacc[blk][u];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- bwd_kv2
//
// Key-stationary backward for rows that fit one query tile (L <= KVTile::CH),
// the mirror image of bwd_q2:
//   workgroup = 4 waves = 64 keys of one (b, h) and a group of n; a wave owns
//   16 keys, whose K and V rows sit in registers as MFMA operands;
//   per n, Q and dO of the slice arrive in LDS by asynchronous copies (same
//   tile layout as K/V, prefetched one slice ahead), lse and delta through
//   LDS as well, and each wave walks all queries 32 at a time:
//     S = Q K^T and dP = dO V^T (lane = key, 4 queries per 16-query block),
//     P = exp(S - lse), dS = P (dP - delta),
//     dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transposed LDS reads),
//     dmask partial = column sums of dS, by an MFMA against a row of ones.
//   The pair-bias columns of the workgroup's 64 keys are read once (through
//   LDS, transposed) and stay in registers for the whole n-group.
template <class T, int D, bool HAS_MASK, bool HAS_PAIR, bool WANT_DMASK>
__global__ __launch_bounds__(256, 2) void evo_bwd_kv2_kernel(BwdArgs a) {
  using TL = KVTile<D>;
  constexpr int KS32 = (D + 31) / 32;
  constexpr bool AUG_PAD = (D % 32) != 0;
  constexpr int NB = TL::CH / 16;    // 16-query blocks per tile
  constexpr int MB = (D + 15) / 16;  // 16-row blocks of dK^T, dV^T
  constexpr int kKeys = 64;
  constexpr int kSlab = HAS_PAIR ? TL::CH * kKeys * 2 : 0;  // pair[:, 64 keys] staged once
  constexpr int kSmem = 2 * TL::BUF_BYTES > kSlab ? 2 * TL::BUF_BYTES : kSlab;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  __shared__ __attribute__((aligned(16))) float slse[2][TL::CH];  // -lse*log2e
  __shared__ __attribute__((aligned(16))) float sdel[2][TL::CH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int L = a.L, H = a.H, N = a.N;
  const int jtiles = (L + kKeys - 1) / kKeys;
  const int ngroups = (N + a.Gq - 1) / a.Gq;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int jt = rest % jtiles;
  rest /= jtiles;
  const int ng = rest % ngroups;
  const int b = rest / ngroups;
  const int j = jt * kKeys + wave * 16 + col;  // this lane's key
  const bool j_valid = j < L;
  const int jc = min(j, L - 1);
  const int n_begin = ng * a.Gq, n_end = min(N, n_begin + a.Gq);
  const int ntiles = n_end - n_begin;

  // ---- pair bias, resident: block qb, lane gets pair[16 qb + 4 g + r][j], r = 0..3
  u32x2 pbias[HAS_PAIR ? NB : 1];
  if constexpr (HAS_PAIR) {
    // stage pair[0..L)[64 keys] row-major (128-byte rows) with 16-byte copies,
    // then read columns with transposed reads
    const uint16_t* pbase = a.pair + ((size_t)b * H + h) * L * L;
    const int kc0 = jt * kKeys;
    for (int base = wave * 64; base < TL::CH * 8; base += 256) {
      const int q = base + lane;
      const int r = q >> 3, c = q & 7;
      const int cc = min(kc0 + 8 * c, L - 8 >= 0 ? L - 8 : 0);
      const uint16_t* src = pbase + (size_t)min(r, L - 1) * L + ((L % 8) == 0 ? cc : 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(smem + base * 16), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if ((L % 8) == 0) {
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        const int row = 16 * qb + 4 * g + (col >> 2);
        const int kcol = wave * 16 + 4 * (col & 3);
        const short4_t v = lds_read_tr_b(smem, (row * kKeys + kcol) * 2);
        pbias[qb] = __builtin_bit_cast(u32x2, v);
      }
    } else {
      const uint16_t* prow = pbase + jc;
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        uint32_t t4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) t4[r] = prow[(size_t)min(16 * qb + 4 * g + r, L - 1) * L];
        pbias[qb][0] = t4[0] | (t4[1] << 16);
        pbias[qb][1] = t4[2] | (t4[3] << 16);
      }
    }
    __syncthreads();
  }

  // ones in row 0 of the column-sum operand
  short8_t ones = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = T::one();
  }

  // ---- per-slice key operands (B of S = Q K^T and dP = dO V^T): lane = key
  short8_t kop[KS32], vop[KS32], kaug;
  short8_t knx[KS32], vnx[KS32];
  uint32_t mnx = 0, mcur = 0;
  float lse_nx = 0.f, del_nx = 0.f;
  auto load_keys = [&](int n) {
    const size_t row = (((size_t)b * N + n) * L + jc) * H + h;
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int d0 = 32 * s + 8 * g;
      short8_t kv = {0, 0, 0, 0, 0, 0, 0, 0}, vv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (d0 + 8 <= D) {
        kv = *reinterpret_cast<const short8_t*>(a.k + row * D + d0);
        vv = *reinterpret_cast<const short8_t*>(a.v + row * D + d0);
      }
      knx[s] = kv;
      vnx[s] = vv;
    }
    if constexpr (HAS_MASK) mnx = a.mask ? a.mask[((size_t)b * N + n) * L + jc] : 0u;
  };
  auto load_rows = [&](int n) {  // lse, delta of query tid
    if (tid < TL::CH) {
      const size_t ri = (((size_t)b * N + n) * H + h) * L + min(tid, L - 1);
      lse_nx = a.lse[ri];
      del_nx = a.delta[ri];
    }
  };
  auto store_rows = [&](int buf) {
    if (tid < TL::CH) {
      // queries past L, or with no finite score, get p = 0
      slse[buf][tid] = (tid < L && lse_nx != kNegInf) ? -lse_nx * kLog2e : kNegInf;
      sdel[buf][tid] = del_nx;
    }
  };

  if (ntiles > 0) {
    load_rows(n_begin);
    issue_kv_tile<D>(smem, a.q, a.dout, ((size_t)b * N + n_begin) * L, 0, L, H, h, wave, lane);
    load_keys(n_begin);
    store_rows(0);
  }
  for (int t = 0; t < ntiles; ++t) {
    const int n = n_begin + t;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      kop[s] = knx[s];
      vop[s] = vnx[s];
    }
    mcur = j_valid ? mnx : (uint32_t)T::kNegInfBits;  // keys past L: masked (not stored anyway)
    // Q' side of the mask product is {s_hi, s_lo}; the key side {m, m'}
    kaug = short8_t{0, 0, 0, 0, 0, 0, 0, 0};
    if (HAS_MASK && ((AUG_PAD && g == D / 8 - 4 * (KS32 - 1)) || (!AUG_PAD && g == 0))) {
      kaug[0] = (short)mcur;
      kaug[1] = (short)(a.s_lo != 0 ? mcur : 0);
    }
    if (AUG_PAD && HAS_MASK) {
      // D = 8, 16: the mask slots follow d inside the last k-step
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (g == D / 8 - 4 * (KS32 - 1)) kop[KS32 - 1][e] = kaug[e];
    }
    if (t + 1 < ntiles) {
      load_rows(n + 1);
      issue_kv_tile<D>(smem + ((t + 1) & 1) * TL::BUF_BYTES, a.q, a.dout, ((size_t)b * N + n + 1) * L, 0, L, H, h,
                       wave, lane);
      load_keys(n + 1);
    }
    const uint8_t* qb_ = smem + (t & 1) * TL::BUF_BYTES;
    const uint8_t* ob_ = qb_ + TL::KCH * 16;
    const float* lrow = slse[t & 1];
    const float* drow = sdel[t & 1];

    // Q (A operand, lane = query row) with {s_hi, s_lo} in the mask slots
    auto qrow_op = [&](int blk, int s) -> short8_t {
      const int r = blk * 16 + col;
      const int c = 4 * s + g;
      short8_t op = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c < TL::KC) {
        op = *reinterpret_cast<const short8_t*>(qb_ + (r * TL::KC + (c ^ kv_swz<TL::KC>(r))) * 16);
      } else if (HAS_MASK && AUG_PAD && c == TL::KC) {
        op[0] = (short)a.s_hi;
        op[1] = (short)a.s_lo;
      }
      return op;
    };
    auto sblk = [&](int blk) -> floatx4 {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS32; ++s) acc = T::mfma16(qrow_op(blk, s), kop[s], acc);
      if constexpr (HAS_MASK && !AUG_PAD) {
        short8_t qa = {0, 0, 0, 0, 0, 0, 0, 0};
        if (g == 0) {
          qa[0] = (short)a.s_hi;
          qa[1] = (short)a.s_lo;
        }
        acc = T::mfma16(qa, kaug, acc);
      }
      return acc;
    };
    auto dpblk = [&](int blk) -> floatx4 {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
      const int r = blk * 16 + col;
#pragma unroll
      for (int s = 0; s < KS32; ++s) {
        const int c = 4 * s + g;
        short8_t op = {0, 0, 0, 0, 0, 0, 0, 0};
        if (c < D / 8) op = *reinterpret_cast<const short8_t*>(ob_ + (r * TL::VC + (c ^ kv_swz<TL::VC>(r))) * 16);
        acc = T::mfma16(op, vop[s], acc);
      }
      return acc;
    };

    floatx4 dk[MB], dv[MB], dmk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      dk[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      dv[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    floatx4 sc[2][2], dp[2][2];
    sc[0][0] = sblk(0);
    sc[0][1] = sblk(1);
    dp[0][0] = dpblk(0);
    dp[0][1] = dpblk(1);
#pragma unroll
    for (int st = 0; st < NB / 2; ++st) {
      if (32 * st < L) {
        const int cur = st & 1;
        if (st + 1 < NB / 2 && 32 * (st + 1) < L) {
          sc[cur ^ 1][0] = sblk(2 * st + 2);
          sc[cur ^ 1][1] = sblk(2 * st + 3);
          dp[cur ^ 1][0] = dpblk(2 * st + 2);
          dp[cur ^ 1][1] = dpblk(2 * st + 3);
        }
        // Q^T and dO^T operands (transposed reads, waited on below)
        short4_t tt[4 * MB];  // [mb][q lo, q hi, o lo, o hi]
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int c0 = 16 * mb + 4 * (col & 3);
          const int r0 = 32 * st + 4 * g + (col >> 2);
          tt[4 * mb + 0] = lds_read_tr_asm(qb_, tr_off<TL::KC>(r0, c0));
          tt[4 * mb + 1] = lds_read_tr_asm(qb_, tr_off<TL::KC>(r0 + 16, c0));
          tt[4 * mb + 2] = lds_read_tr_asm(ob_, tr_off<TL::VC>(r0, c0));
          tt[4 * mb + 3] = lds_read_tr_asm(ob_, tr_off<TL::VC>(r0 + 16, c0));
        }
        float pv[2][4], ds[2][4];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int blk = 2 * st + hb;
          const floatx4 nl4 = *reinterpret_cast<const floatx4*>(lrow + 16 * blk + 4 * g);
          const floatx4 dl4 = *reinterpret_cast<const floatx4*>(drow + 16 * blk + 4 * g);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float s;
            if constexpr (HAS_PAIR) {
              const uint32_t w = pbias[blk][r / 2];
              s = (r & 1) ? T::fma_mix_hi(sc[cur][hb][r], a.scale, w) : T::fma_mix_lo(sc[cur][hb][r], a.scale, w);
            } else {
              s = sc[cur][hb][r] * a.scale;
            }
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, kLog2e, nl4[r]));
            pv[hb][r] = p;
            ds[hb][r] = p * (dp[cur][hb][r] - dl4[r]);
          }
        }
        const short8_t pb = __builtin_bit_cast(
            short8_t, u32x4{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]), T::pack2(pv[1][0], pv[1][1]),
                            T::pack2(pv[1][2], pv[1][3])});
        const short8_t db = __builtin_bit_cast(
            short8_t, u32x4{T::pack2(ds[0][0], ds[0][1]), T::pack2(ds[0][2], ds[0][3]), T::pack2(ds[1][0], ds[1][1]),
                            T::pack2(ds[1][2], ds[1][3])});
        if constexpr (WANT_DMASK) dmk = T::mfma16(ones, db, dmk);
        lds_wait_all(tt);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          dk[mb] = T::mfma16(cat4(tt[4 * mb], tt[4 * mb + 1]), db, dk[mb]);
          dv[mb] = T::mfma16(cat4(tt[4 * mb + 2], tt[4 * mb + 3]), pb, dv[mb]);
        }
      }
    }
    // ---- dK = scale * dK^T, dV: lane holds d = 16 mb + 4 g + 0..3 of key j
    if (j_valid) {
      const size_t row = (((size_t)b * N + n) * L + j) * H + h;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int d = 16 * mb + 4 * g;
        if (d < D) {
          u32x2 wk, wv;
          wk[0] = T::pack2(dk[mb][0] * a.scale, dk[mb][1] * a.scale);
          wk[1] = T::pack2(dk[mb][2] * a.scale, dk[mb][3] * a.scale);
          wv[0] = T::pack2(dv[mb][0], dv[mb][1]);
          wv[1] = T::pack2(dv[mb][2], dv[mb][3]);
          *reinterpret_cast<u32x2*>(a.dk + row * D + d) = wk;
          *reinterpret_cast<u32x2*>(a.dv + row * D + d) = wv;
        }
      }
      if (WANT_DMASK && g == 0) a.dmask_part[(((size_t)b * N + n) * H + h) * L + j] = dmk[0];
    }
    if (t + 1 < ntiles) store_rows((t + 1) & 1);
  }
}

// ---------------------------------------------------------------- bwd_fin

// Bias-gradient reductions in one launch.  Threads [0, n_pair) sum the dpair
// partials of the n-groups (4 consecutive elements each when the element
// count allows 16-byte access); the rest sum the per-head dmask partials.
// Both sums run in a fixed order, so the result is bitwise reproducible.
template <class T, bool VEC>
__global__ __launch_bounds__(256) void evo_bwd_fin_kernel(BwdArgs a, int ngroups, int from_f32, int64_t n_pair,
                                                          int64_t n_mask) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n_pair) {
    const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
    if constexpr (VEC) {
      const int64_t idx = 4 * e;
      floatx4 s;
      if (from_f32) {
        s = *reinterpret_cast<const floatx4*>(a.dpair_f32 + idx);
      } else {
        floatx4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        int gg = 0;
        for (; gg + 1 < ngroups; gg += 2) {
          s0 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)gg * per + idx);
          s1 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)(gg + 1) * per + idx);
        }
        if (gg < ngroups) s0 += *reinterpret_cast<const floatx4*>(a.dpair_part + (int64_t)gg * per + idx);
        s = s0 + s1;
        *reinterpret_cast<floatx4*>(a.dpair_f32 + idx) = s;
      }
      u32x2 w;
      w[0] = T::pack2(s[0], s[1]);
      w[1] = T::pack2(s[2], s[3]);
      *reinterpret_cast<u32x2*>(a.dpair + idx) = w;
    } else {
      float s;
      if (from_f32) {
        s = a.dpair_f32[e];
      } else {
        float s0 = 0.f, s1 = 0.f;
        int gg = 0;
        for (; gg + 1 < ngroups; gg += 2) {
          s0 += a.dpair_part[(int64_t)gg * per + e];
          s1 += a.dpair_part[(int64_t)(gg + 1) * per + e];
        }
        if (gg < ngroups) s0 += a.dpair_part[(int64_t)gg * per + e];
        s = s0 + s1;
        a.dpair_f32[e] = s;
      }
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
  }
}

__global__ __launch_bounds__(256) void evo_zero_f32_kernel(float* p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0.f;
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HM, bool HP>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const bool want_dmask = a.dmask != nullptr;
  const bool want_dpair = a.dpair != nullptr;
  const int nchunks = (a.L + kQChunk - 1) / kQChunk;
  const bool fits = a.L <= KVTile<D>::CH;
  // ragged rows without a user mask take the mask path (zero mask, keys past L at -inf)
  const bool hm_eff = HM || (a.L % 32) != 0;
  if (fits) {
    // bwd_q2 forms delta itself and leaves it in the workspace for bwd_kv2
    const int grid2 = a.B * a.H * ((a.L + kQ2Rows - 1) / kQ2Rows) * a.n_groups_q;
    prof_begin(K_BWD_Q, st);
    if (hm_eff) {
      if (want_dpair)
        hipLaunchKernelGGL((evo_bwd_q2_kernel<T, D, true, HP, true>), dim3(grid2), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((evo_bwd_q2_kernel<T, D, true, HP, false>), dim3(grid2), dim3(256), 0, st, a);
    } else {
      if (want_dpair)
        hipLaunchKernelGGL((evo_bwd_q2_kernel<T, D, false, HP, true>), dim3(grid2), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((evo_bwd_q2_kernel<T, D, false, HP, false>), dim3(grid2), dim3(256), 0, st, a);
    }
    prof_end(K_BWD_Q, st);
    const int gridk = a.B * a.H * ((a.L + 63) / 64) * ((a.N + a.Gq - 1) / a.Gq);
    prof_begin(K_BWD_KV, st);
    if (hm_eff) {
      if (want_dmask)
        hipLaunchKernelGGL((evo_bwd_kv2_kernel<T, D, true, HP, true>), dim3(gridk), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((evo_bwd_kv2_kernel<T, D, true, HP, false>), dim3(gridk), dim3(256), 0, st, a);
    } else {
      hipLaunchKernelGGL((evo_bwd_kv2_kernel<T, D, false, HP, false>), dim3(gridk), dim3(256), 0, st, a);
    }
    prof_end(K_BWD_KV, st);
  } else {
    {
      const int64_t rows = (int64_t)a.B * a.N * a.L * a.H;
      prof_begin(K_BWD_PRE, st);
      hipLaunchKernelGGL((evo_bwd_pre_kernel<T, D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, a);
      prof_end(K_BWD_PRE, st);
    }
    {
      const int grid = a.B * a.N * a.H * ((a.L + kKvKeys - 1) / kKvKeys);
      prof_begin(K_BWD_KV, st);
      if (want_dmask)
        hipLaunchKernelGGL((evo_bwd_kv_kernel<T, D, HM, HP, true>), dim3(grid), dim3(256), 0, st, a);
      else
        hipLaunchKernelGGL((evo_bwd_kv_kernel<T, D, HM, HP, false>), dim3(grid), dim3(256), 0, st, a);
      prof_end(K_BWD_KV, st);
    }
    {
      const int grid = a.B * a.H * ((a.L + 31) / 32) * a.n_groups_q;
      if (want_dpair && nchunks > 6) {
        const int64_t n = (int64_t)a.B * a.H * a.L * a.L;
        hipLaunchKernelGGL(evo_zero_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.dpair_f32, n);
      }
      prof_begin(K_BWD_Q, st);
      if (!want_dpair) {
        hipLaunchKernelGGL((evo_bwd_q_kernel<T, D, HM, HP, false, 0>), dim3(grid), dim3(256), 0, st, a);
      } else if (nchunks <= 2) {
        hipLaunchKernelGGL((evo_bwd_q_kernel<T, D, HM, HP, true, 2>), dim3(grid), dim3(256), 0, st, a);
      } else if (nchunks <= 4) {
        hipLaunchKernelGGL((evo_bwd_q_kernel<T, D, HM, HP, true, 4>), dim3(grid), dim3(256), 0, st, a);
      } else if (nchunks <= 6) {
        hipLaunchKernelGGL((evo_bwd_q_kernel<T, D, HM, HP, true, 6>), dim3(grid), dim3(256), 0, st, a);
      } else {
        hipLaunchKernelGGL((evo_bwd_q_kernel<T, D, HM, HP, true, 0>), dim3(grid), dim3(256), 0, st, a);
      }
      prof_end(K_BWD_Q, st);
    }
  }
  if (want_dmask || want_dpair) {
    const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
    const bool vec = (per % 4) == 0;
    const int64_t n_pair = want_dpair ? (vec ? per / 4 : per) : 0;
    const int64_t n_mask = want_dmask ? (int64_t)a.B * a.N * a.L : 0;
    const int from_f32 = (!fits && nchunks > 6) ? 1 : 0;
    const unsigned blocks = (unsigned)((n_pair + n_mask + 255) / 256);
    prof_begin(K_BWD_FIN, st);
    if (vec)
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, true>), dim3(blocks), dim3(256), 0, st, a, a.n_groups_q, from_f32,
                         n_pair, n_mask);
    else
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, false>), dim3(blocks), dim3(256), 0, st, a, a.n_groups_q, from_f32,
                         n_pair, n_mask);
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
