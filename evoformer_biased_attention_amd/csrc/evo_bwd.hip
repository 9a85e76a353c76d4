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
// keys; dpair over n; dmask over heads and queries), so the work is split over
// two kernels that each recompute P (bwd_q3, bwd_kv3 in evo_bwd_tile.hip) and
// the reduction kernel of this file:
//   bwd_fin  dmask = sum_h partials, dpair = sum_g partials, dQ = sum of the
//            key-tile partials (rows longer than one key tile), each in a
//            fixed order (bitwise reproducible), then rounded to dtype.
// Rows longer than one key tile go through bwd_q3 in chunks of slices so that
// the partials stay within a fixed budget: each chunk's dQ partials are summed
// by a bwd_fin launch of their own, and the dpair group slots carry their sums
// from chunk to chunk (bwd_q3 of a later chunk continues them), so the last
// bwd_fin sums the slots once.
#include <algorithm>

#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

// ---------------------------------------------------------------- bwd_fin

// Reductions in one launch, each in a fixed order (bitwise reproducible):
//   threads [0, n_pair)                  dpair = sum of the n-group partials
//                                        (4 consecutive elements each when
//                                        the count allows 16-byte access);
//   [n_pair, n_pair + n_mask)            dmask = sum of the per-head partials;
//   [n_pair + n_mask, ... + n_dq)        dQ = sum of the key-tile partials
//                                        (rows longer than one key tile), 4
//                                        consecutive elements each.
// Sum of the n partials src[g * per] in a fixed order, with up to 32 loads in
// flight per thread (the sum is bound by memory latency, not by the adds;
// 32 against 16: C2's bwd_fin -4.6%, the same bits).
template <class V>
__device__ __forceinline__ V sum_partials(const V* src, int64_t per, int n) {
  V acc[4] = {V{}, V{}, V{}, V{}};
  int g = 0;
  for (; g + 32 <= n; g += 32) {
    V t[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) t[u] = src[(int64_t)(g + u) * per];
#pragma unroll
    for (int u = 0; u < 32; ++u) acc[u & 3] += t[u];
  }
  for (; g + 16 <= n; g += 16) {
    V t[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) t[u] = src[(int64_t)(g + u) * per];
#pragma unroll
    for (int u = 0; u < 16; ++u) acc[u & 3] += t[u];
  }
  for (; g + 4 <= n; g += 4) {
    V t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = src[(int64_t)(g + u) * per];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] += t[u];
  }
  for (; g < n; ++g) acc[0] += src[(int64_t)g * per];
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <class T, bool VEC>
__global__ __launch_bounds__(256) void evo_bwd_fin_kernel(BwdArgs a, int ngroups, int64_t n_pair, int64_t n_mask,
                                                          int64_t n_dq, int jtiles, int D) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n_pair) {
    const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
    if constexpr (VEC) {
      const int64_t idx = 4 * e;
      const floatx4 s = sum_partials(reinterpret_cast<const floatx4*>(a.dpair_part) + e, per / 4, ngroups);
      *reinterpret_cast<floatx4*>(a.dpair_f32 + idx) = s;
      u32x2 w;
      w[0] = T::pack2(s[0], s[1]);
      w[1] = T::pack2(s[2], s[3]);
      *reinterpret_cast<u32x2*>(a.dpair + idx) = w;
    } else {
      const float s = sum_partials(a.dpair_part + e, per, ngroups);
      a.dpair_f32[e] = s;
      a.dpair[e] = T::from_f32(s);
    }
    return;
  }
  const int64_t m = e - n_pair;
  if (m < n_mask) {
    const int j = (int)(m % a.L);
    const int64_t bn = m / a.L;
    const float s = sum_partials(a.dmask_part + bn * a.H * a.L + j, (int64_t)a.L, a.H);
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
    // the partials are dense [B,N,L,H,D]; dQ has the strides of the call
    // (the chunk's slices q_n0 .. q_n0 + q_nc - 1)
    const int64_t hd = idx % ((int64_t)a.H * D), r = idx / ((int64_t)a.H * D);
    const int64_t l = r % a.L, bn = r / a.L;
    const int64_t dst = (bn / a.q_nc) * a.sB + (a.q_n0 + bn % a.q_nc) * a.sN + l * a.sL + hd;
    *reinterpret_cast<u32x2*>(a.dq + dst) = w;
  }
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HM, bool HP>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  const bool want_dmask = a.dmask != nullptr;
  const bool want_dpair = a.dpair != nullptr;
  const bool fits = a.L <= KVTile<D>::CH;
  const int jtiles = (a.L + KVTile<D>::CH - 1) / KVTile<D>::CH;
  const int64_t per = (int64_t)a.B * a.H * a.L * a.L;
  const bool vec = (per % 4) == 0;
  const int slots = a.n_groups_q;  // dpair group slots (those of a full chunk)
  auto fin = [&](const BwdArgs& af, int64_t n_pair, int64_t n_mask, int64_t n_dq) {
    if (n_pair + n_mask + n_dq == 0) return;
    const unsigned blocks = (unsigned)((n_pair + n_mask + n_dq + 255) / 256);
    prof_begin(K_BWD_FIN, st);
    if (vec)
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, true>), dim3(blocks), dim3(256), 0, st, af, slots, n_pair, n_mask,
                         n_dq, jtiles, D);
    else
      hipLaunchKernelGGL((evo_bwd_fin_kernel<T, false>), dim3(blocks), dim3(256), 0, st, af, slots, n_pair, n_mask,
                         n_dq, jtiles, D);
    prof_end(K_BWD_FIN, st);
  };
  const int64_t n_pair = want_dpair ? (vec ? per / 4 : per) : 0;
  const int64_t n_mask = want_dmask ? (int64_t)a.B * a.N * a.L : 0;
  const bool bf16 = std::is_same<T, BF16>::value;
  if (fits) {
    const hipError_t e = launch_bwd_tile(a, D, bf16, st);
    if (e != hipSuccess) return e;
    fin(a, n_pair, n_mask, 0);
  } else if (!HP) {
    // no pair bias: bwd_q3 walks every key tile of its slices with dQ in
    // registers (no partials), then bwd_kv3 over query tiles (it reads delta)
    // and the sums of the dmask partials
    hipError_t e = launch_bwd_q_split(a, D, bf16, 2, st);
    if (e != hipSuccess) return e;
    if ((e = launch_bwd_q_split(a, D, bf16, 1, st)) != hipSuccess) return e;
    fin(a, 0, n_mask, 0);
  } else {
    // per chunk of slices: bwd_q3 over its key tiles (dQ partials, delta,
    // dpair slot sums), then the sum of its dQ partials; after the last
    // chunk bwd_kv3 over query tiles (it reads delta) and the final sums
    const int chunks = (a.N + a.q_nc - 1) / a.q_nc;
    for (int c = 0; c < chunks; ++c) {
      BwdArgs ac = a;
      ac.q_n0 = c * a.q_nc;
      ac.q_nc = std::min(a.q_nc, a.N - ac.q_n0);
      ac.n_groups_q = (ac.q_nc + a.Gq - 1) / a.Gq;
      ac.dpair_carry = c > 0;
      hipError_t e = launch_bwd_q_split(ac, D, bf16, 0, st);
      if (e != hipSuccess) return e;
      const int64_t n_dq = (int64_t)a.B * ac.q_nc * a.L * a.H * D / 4;
      if (c + 1 < chunks) {
        fin(ac, 0, 0, n_dq);
      } else {
        if ((e = launch_bwd_q_split(a, D, bf16, 1, st)) != hipSuccess) return e;
        fin(ac, n_pair, n_mask, n_dq);
      }
    }
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
