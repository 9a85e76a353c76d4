// Fused forward of Evoformer biased attention on gfx950.
//
// Computes, per (b, n, h) slice, O = softmax_j(scale*QK^T + mask + pair) V and
// the natural-log log-sum-exp of every query row (DeepSpeed4Science guide,
// §3.5 for the operation, §3.7 for the saved fp32 lse).  The score matrix is
// never written out: keys are streamed in chunks and the row softmax is
// carried online (running max and running sum), so the slice costs O(L) state
// per query row.
//
// Work decomposition
//   workgroup = 4 waves = 128 query rows of one (b, h) and a group of G
//               consecutive n; each wave owns 32 query rows.
//   For every n of the group, K and V are staged chunk by chunk in LDS, and
//   each wave walks the keys 32 at a time with two MFMA products:
//     S^T = K Q^T  (keys x queries, so a lane owns one query row), and
//     O^T += V^T P^T, with P^T taken straight from the S^T accumulator and V^T
//     fetched from LDS by transposed reads.
//   The pair bias does not depend on n.  When a row of it fits in registers
//   (L <= 256) each wave loads its 32 rows once and reuses them for all G
//   slices; otherwise it is re-read from L2 for every block.
//   The mask bias enters the QK^T product itself: K gets extra columns holding
//   mask[j] and Q gets sqrt(D) split into two 16-bit parts, so the MFMA adds
//   mask[j]*sqrt(D), which the scale turns back into mask[j].
//   Running max: the exponent base is only moved when a row's block max
//   exceeds it by more than 8 (log2 units), so exp values stay below 2^8 and
//   the accumulator is rarely rescaled.
#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

constexpr int kFwdWaves = 4;
constexpr int kFwdRows = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdChunk = 128;            // keys staged in LDS at a time
constexpr float kTauNat = 5.545177444479562f;  // 8 * ln 2

template <int D, bool HAS_MASK>
struct FwdShape {
  static constexpr int KSTEPS_D = (D + 15) / 16;
  static constexpr bool AUG_IN_PAD = (D % 16) != 0;
  static constexpr int KSTEPS = KSTEPS_D + ((HAS_MASK && !AUG_IN_PAD) ? 1 : 0);
  static constexpr int KW = KSTEPS * 16;  // logical K/Q row width incl. mask columns
  static constexpr int KS = padded_stride_elems(KW);
  static constexpr int VW = D < 32 ? 32 : D;  // columns the transposed reads touch
  static constexpr int VS = (VW == 64) ? 80 : VW;
  static constexpr int MB = (D + 31) / 32;  // 32-row blocks of O^T
};

// Load 8 consecutive 16-bit values of a global row; columns >= D come from the
// mask-augmentation pattern (or zero).
template <int D>
__device__ __forceinline__ short8_t load_q8(const uint16_t* row, int c, bool valid, uint16_t s_hi, uint16_t s_lo,
                                            bool has_mask) {
  short8_t r = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c + 8 <= D) {
    if (valid) r = *reinterpret_cast<const short8_t*>(row + c);
  } else if (has_mask) {
    for (int e = 0; e < 8; ++e) {
      int a = c + e - D;
      r[e] = (short)(a == 0 ? s_hi : (a == 1 ? s_lo : 0));
    }
  }
  return r;
}

// Pair-bias values for one 32-key block in the S^T accumulator layout:
// lane (query i) gets pair[i][j0 + 8q + 4*(l/32) + u], q,u = 0..3, packed two per dword.
__device__ __forceinline__ void load_pair_block(u32x2 (&dst)[4], const uint16_t* prow, int i_valid, int j0, int L,
                                                int half, bool vec_ok) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int j = j0 + 8 * q + 4 * half;
    u32x2 v = {0u, 0u};
    if (i_valid) {
      if (vec_ok && j + 4 <= L) {
        v = *reinterpret_cast<const u32x2*>(prow + j);
      } else {
        uint16_t t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = (j + u < L) ? prow[j + u] : (uint16_t)0;
        v[0] = (uint32_t)t[0] | ((uint32_t)t[1] << 16);
        v[1] = (uint32_t)t[2] | ((uint32_t)t[3] << 16);
      }
    }
    dst[q] = v;
  }
}

__device__ __forceinline__ uint16_t pick16(const u32x2 (&b)[4], int r) {
  uint32_t w = b[r / 4][(r % 4) / 2];
  return (r & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xffffu);
}

template <class T, int D, bool HAS_MASK, bool HAS_PAIR, int RES>
__global__ __launch_bounds__(256, 2) void evo_fwd_kernel(FwdArgs a) {
  using S = FwdShape<D, HAS_MASK>;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kFwdChunk * S::KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kFwdChunk * S::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int L = a.L, H = a.H, N = a.N;

  // workgroup -> (b, h, i-tile, n-group); consecutive ids of one XCD share (b, h, i-tile)
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int ng = wg % a.n_groups;
  int rest = wg / a.n_groups;
  const int it = rest % a.i_tiles;
  rest /= a.i_tiles;
  const int h = rest % H;
  const int b = rest / H;

  const int i = it * kFwdRows + wave * 32 + (lane & 31);
  const bool i_valid = i < L;
  const int n_begin = ng * a.G;
  const int n_end = min(N, n_begin + a.G);
  const int nkb = (L + 31) / 32;  // key blocks

  // ---- pair-bias registers (loaded once when the whole row fits)
  u32x2 pres[RES > 0 ? RES : 1][4];
  const uint16_t* prow = nullptr;
  const bool pvec = (L % 4) == 0;
  if constexpr (HAS_PAIR) {
    prow = a.pair + (((size_t)b * H + h) * L + (i_valid ? i : 0)) * L;
    if constexpr (RES > 0) {
#pragma unroll
      for (int kb = 0; kb < RES; ++kb) {
        if (kb < nkb) load_pair_block(pres[kb], prow, i_valid, kb * 32, L, half, pvec);
      }
    }
  }

  for (int n = n_begin; n < n_end; ++n) {
    const size_t slice = ((size_t)b * N + n) * L;  // row index of (b, n, 0)
    // ---- Q operand (B of S^T = K Q^T): lane owns query i, 8 columns per k-step
    short8_t qop[S::KSTEPS];
    {
      const uint16_t* qrow = a.q + ((slice + (i_valid ? i : 0)) * H + h) * D;
#pragma unroll
      for (int s = 0; s < S::KSTEPS; ++s)
        qop[s] = load_q8<D>(qrow, 16 * s + 8 * half, i_valid, a.s_hi, a.s_lo, HAS_MASK);
    }
    floatx16 oacc[S::MB];
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) oacc[mb] = floatx16{};
    float m_used = kNegInf;
    float l_part = 0.f;

    // ---- stage K (with mask columns) and V rows [kc0, kc0 + chunk) of slice n
    auto stage = [&](const int kc0, const size_t slice_, const int n_) {
      constexpr int V8 = D / 8;  // 16-byte pieces per row
      for (int t = tid; t < kFwdChunk * V8; t += 256) {
        int r = t / V8, c8 = t % V8;
        int j = kc0 + r;
        short8_t kv = {0, 0, 0, 0, 0, 0, 0, 0}, vv = {0, 0, 0, 0, 0, 0, 0, 0};
        if (j < L) {
          size_t off = ((slice_ + j) * H + h) * D + c8 * 8;
          kv = *reinterpret_cast<const short8_t*>(a.k + off);
          vv = *reinterpret_cast<const short8_t*>(a.v + off);
        }
        *reinterpret_cast<short8_t*>(&sK[r * S::KS + c8 * 8]) = kv;
        *reinterpret_cast<short8_t*>(&sV[r * S::VS + c8 * 8]) = vv;
      }
      if constexpr (S::KW > D) {
        for (int r = tid; r < kFwdChunk; r += 256) {
          int j = kc0 + r;
          uint16_t m = 0;
          if constexpr (HAS_MASK) m = (j < L) ? a.mask[((size_t)b * N + n_) * L + j] : (uint16_t)0;
          for (int c = D; c < S::KW; ++c) {
            uint16_t val = 0;
            if (HAS_MASK && c == D) val = m;
            if (HAS_MASK && c == D + 1 && a.s_lo != 0) val = m;
            sK[r * S::KS + c] = val;
          }
        }
      }
    };

    // ---- one 32-key block: scores, online softmax, PV
    auto block = [&](const int jb, const int j0, const u32x2 (&pb)[4]) {
      floatx16 acc = floatx16{};
#pragma unroll
      for (int s = 0; s < S::KSTEPS; ++s) {
        short8_t kop = *reinterpret_cast<const short8_t*>(&sK[(jb * 32 + (lane & 31)) * S::KS + 16 * s + 8 * half]);
        acc = T::mfma(kop, qop[s], acc);
      }
      float sv[16];
      if constexpr (HAS_PAIR) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = T::fma_mix(acc[r], a.scale, pick16(pb, r));
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[r] = acc[r] * a.scale;
      }
      if (j0 + 32 > L) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int j = j0 + 8 * (r / 4) + 4 * half + (r % 4);
          if (j >= L) sv[r] = kNegInf;
        }
      }
      float mb = sv[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mb = __builtin_fmaxf(mb, sv[r]);
      mb = xhalf_max(mb);
      const bool need = mb > m_used + kTauNat;
      if (__builtin_amdgcn_ballot_w64(need)) {
        float m_new = need ? mb : m_used;
        float alpha = need ? __builtin_amdgcn_exp2f((m_used - m_new) * kLog2e) : 1.f;
        m_used = m_new;
        l_part *= alpha;
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[mb2][r] *= alpha;
      }
      const float neg_ml = (m_used == kNegInf) ? 0.f : -m_used * kLog2e;
      uint32_t pk[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], kLog2e, neg_ml));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r + 1], kLog2e, neg_ml));
        l_part += p0 + p1;
        pk[r / 2] = T::pack2(p0, p1);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        short8_t bop = __builtin_bit_cast(short8_t, u32x4{pk[4 * t], pk[4 * t + 1], pk[4 * t + 2], pk[4 * t + 3]});
        const int qg = lane >> 4, i16 = lane & 15;
        const int g = qg >> 1;
        const int k0 = jb * 32 + 16 * t + 4 * g;
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2) {
          const int n0 = 16 * (qg & 1) + 32 * mb2;
          const int e1 = (k0 + (i16 >> 2)) * S::VS + n0 + 4 * (i16 & 3);
          const int e2 = e1 + 8 * S::VS;
          short8_t aop = cat4(lds_read_tr(sV, e1), lds_read_tr(sV, e2));
          oacc[mb2] = T::mfma(aop, bop, oacc[mb2]);
        }
      }
    };

    const int nchunks = (L + kFwdChunk - 1) / kFwdChunk;
    if constexpr (RES > 0) {
      // L <= 32*RES: the chunk and block loops are unrolled so that the
      // resident pair-bias block is selected at compile time.
      constexpr int kChunksRes = (RES * 32 + kFwdChunk - 1) / kFwdChunk;
#pragma unroll
      for (int c = 0; c < kChunksRes; ++c) {
        if (c < nchunks) {
          const int kc0 = c * kFwdChunk;
          __syncthreads();  // previous chunk fully consumed
          stage(kc0, slice, n);
          __syncthreads();
#pragma unroll
          for (int jb = 0; jb < kFwdChunk / 32; ++jb) {
            const int kb = c * (kFwdChunk / 32) + jb;
            if (kb < RES && kc0 + jb * 32 < L) block(jb, kc0 + jb * 32, pres[kb < RES ? kb : 0]);
          }
        }
      }
    } else {
      for (int c = 0; c < nchunks; ++c) {
        const int kc0 = c * kFwdChunk;
        __syncthreads();
        stage(kc0, slice, n);
        __syncthreads();
        const int nblk = (min(kFwdChunk, L - kc0) + 31) / 32;
        for (int jb = 0; jb < nblk; ++jb) {
          u32x2 pb[4] = {};
          if constexpr (HAS_PAIR) load_pair_block(pb, prow, i_valid, kc0 + jb * 32, L, half, pvec);
          block(jb, kc0 + jb * 32, pb);
        }
      }
    }

    // ---- epilogue: normalise, store O and lse
    const float l_tot = xhalf_sum(l_part);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (i_valid) {
      uint16_t* orow = a.out + ((slice + i) * H + h) * D;
#pragma unroll
      for (int mb2 = 0; mb2 < S::MB; ++mb2)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d = 32 * mb2 + 8 * q + 4 * half;
          if (d < D) {
            u32x2 w;
            w[0] = T::pack2(oacc[mb2][4 * q] * inv, oacc[mb2][4 * q + 1] * inv);
            w[1] = T::pack2(oacc[mb2][4 * q + 2] * inv, oacc[mb2][4 * q + 3] * inv);
            *reinterpret_cast<u32x2*>(orow + d) = w;
          }
        }
      if (half == 0) {
        float lse = (m_used == kNegInf || !(l_tot > 0.f)) ? kNegInf : m_used + __logf(l_tot);
        a.lse[(((size_t)b * N + n) * H + h) * L + i] = lse;
      }
    }
  }
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HM, bool HP>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int grid = a.B * a.H * a.i_tiles * a.n_groups;
  prof_begin(K_FWD, stream);
  if (HP && a.L <= 256) {
    hipLaunchKernelGGL((evo_fwd_kernel<T, D, HM, HP, 8>), dim3(grid), dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((evo_fwd_kernel<T, D, HM, HP, 0>), dim3(grid), dim3(256), 0, stream, a);
  }
  prof_end(K_FWD, stream);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  const bool hm = a.mask != nullptr, hp = a.pair != nullptr;
  if (hm && hp) return launch_fwd_t<T, D, true, true>(a, s);
  if (hm) return launch_fwd_t<T, D, true, false>(a, s);
  if (hp) return launch_fwd_t<T, D, false, true>(a, s);
  return launch_fwd_t<T, D, false, false>(a, s);
}

template <class T>
static hipError_t launch_fwd_dt(const FwdArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 8: return launch_fwd_d<T, 8>(a, s);
    case 16: return launch_fwd_d<T, 16>(a, s);
    case 32: return launch_fwd_d<T, 32>(a, s);
    case 64: return launch_fwd_d<T, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(FwdArgs a, int D, bool bf16, hipStream_t stream) {
  a.i_tiles = (a.L + kFwdRows - 1) / kFwdRows;
  a.n_groups = (a.N + a.G - 1) / a.G;
  return bf16 ? launch_fwd_dt<BF16>(a, D, stream) : launch_fwd_dt<F16>(a, D, stream);
}

}  // namespace evo
