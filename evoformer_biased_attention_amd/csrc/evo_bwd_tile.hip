// Backward of Evoformer biased attention, gfx950: the query-side and key-side
// tile kernels (rows of one key tile, L <= 256 or L <= 128 at D = 64, and,
// with SPLIT / MULTI, longer rows).
//
// DeepSpeed4Science guide §3.7: recompute P from the saved fp32 lse, derive
// delta = rowsum(dO * O), then dQ, dK, dV and the two bias gradients, the bias
// gradients accumulated in fp32:
//   P = exp(S - lse),  dS = P (dP - delta),  dP = dO V^T
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
//   dmask[b,n,j] = sum_h sum_i dS,  dpair[b,h,i,j] = sum_n dS
//
// Two kernels, each recomputing S and P (the reductions run along different
// axes and stay on chip without atomics):
//   bwd_q3   128 queries of one (b, h) and a group of n per workgroup: dQ,
//            delta (written for bwd_kv3), and dpair summed over the n-group in
//            registers, written once per group as an fp32 partial;
//   bwd_kv3  128 keys of one (b, h) and a group of n per workgroup: dK, dV and
//            the per-head dmask partials.
// Both use v_mfma_f32_16x16x32 tiles (a wave owns 16 rows) and take as much
// per-score work off the vector ALU as the accumulator layout allows:
//   - the mask enters the score MFMA as its accumulator input (sqrt(D) * mask,
//     -inf for keys past L), so it costs neither a VALU op nor an MFMA;
//   - -delta enters the dP MFMA the same way, so dS = P * acc is one multiply;
//   - the n-sum of dpair is an MFMA against an identity operand (fp16; bf16
//     adds the fp32 dS in place);
//   - LDS operand reads use the instruction's immediate offset field;
//   - keys masked with -inf have P = dS = 0: bwd_q3 stops a slice's steps at
//     the tile's last key that is not -inf (the padding at the end of a row
//     is not computed), and a bwd_kv3 wave whose 16 keys all are -inf skips
//     the slice and writes zeros.
// Per score the vector ALU then does: the bias add (fused with the scale),
// the exp argument, the exp, dS = P * acc and a share of the 16-bit packing.
#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

// A workgroup has NW waves; wave w owns rows 16w..16w+15 of the workgroup's
// 16 NW queries (bwd_q3) or keys (bwd_kv3).  Eight waves (128 rows) halve the
// tile traffic per score against four and still keep two waves per SIMD.
constexpr int kWaves = 8;

// Per-thread byte offsets, relative to the first element of a (b, n) slice,
// of the 16-byte chunks this thread copies into a tile (rows = keys
// [kc0, kc0 + CH), clamped to L - 1, sL elements apart; K-layout chunks first,
// then V-layout chunks).  They do not depend on n, so the per-slice copy is a
// base pointer plus these offsets.
template <int D, int NT>
struct TileCopy {
  static constexpr int N = (KVTile<D>::TCH + NT - 1) / NT;  // chunks per thread (the last may be partial)
  uint32_t off[N];
};

template <int D, int NT>
__device__ __forceinline__ void tile_chunk_offsets(TileCopy<D, NT>& tc, int kc0, int L, int64_t sL, int h,
                                                   int wave, int lane) {
  using TL = KVTile<D>;
#pragma unroll
  for (int c = 0; c < TileCopy<D, NT>::N; ++c) {
    const int q = min(wave * 64 + NT * c + lane, TL::TCH - 1);
    int r, cc;
    if (q < TL::KCH) {
      r = q / TL::KC;
      cc = (q % TL::KC) ^ kv_swz<TL::KC>(r);
    } else {
      const int q2 = q - TL::KCH;
      r = q2 / TL::VC;
      cc = (q2 % TL::VC) ^ kv_swz<TL::VC>(r);
      if (cc >= D / 8) cc = 0;  // columns the transposed reads touch but never use
    }
    const int j = min(kc0 + r, L - 1);
    tc.off[c] = (uint32_t)((j * sL + h * D + 8 * cc) * 2);
  }
}

// Issue the asynchronous copies of one slice's tile (rows of `kx` in the K
// layout, rows of `vx` in the V layout) into an LDS buffer.
template <int D, int NT>
__device__ __forceinline__ void issue_tile(uint8_t* buf, const uint16_t* kx, const uint16_t* vx,
                                           const TileCopy<D, NT>& tc, int wave) {
  using TL = KVTile<D>;
#pragma unroll
  for (int c = 0; c < TileCopy<D, NT>::N; ++c) {
    const int base = wave * 64 + NT * c;  // wave-uniform
    if ((TL::TCH % NT) != 0 && base >= TL::TCH) break;
    const char* src = reinterpret_cast<const char*>(base < TL::KCH ? kx : vx) + tc.off[c];
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(buf + base * 16), 16, 0, 0);
  }
}

// ---------------------------------------------------------------- bwd_q3
//
// Wave w owns queries 16w..16w+15 of the tile (lane = query, S^T layout).
// Per n the K and V rows of the slice arrive in LDS (double-buffered,
// prefetched one slice ahead); per 32-key step:
//   S^T  = K Q^T + sqrt(D) mask          (mask as accumulator input)
//   dP^T = V dO^T - delta                (-delta as accumulator input)
//   P = exp2((S*scale + pair) log2e - lse log2e),  dS^T = P dP^T
//                                        (bf16: sqrt(D) pair enters S^T by a
//                                        16x16x16 MFMA against sqrt(D) I)
//   dQ^T += K^T dS^T                     (K^T by transposed LDS reads)
//   dpair^T[block] += I dS^T[block]      (16x16x16 MFMA against an identity)
template <class T, int D, bool HAS_PAIR, bool WANT_DPAIR, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW) void evo_bwd_q3_kernel(BwdArgs a) {
  using TL = KVTile<D>;
  constexpr int KS32 = (D + 31) / 32;  // 32-wide k-steps over d
  constexpr int NB = TL::CH / 16;      // 16-key blocks per tile
  constexpr int NSTEP = TL::CH / 32;   // 32-key steps per tile
  constexpr int MB = (D + 15) / 16;    // 16-row blocks of dQ^T
  constexpr int KC = TL::KC, VC = TL::VC;
  constexpr int NT = 64 * NW, kRows = 16 * NW;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) float smk[2][TL::CH];  // sqrt(D) * mask of key j, -inf past L
  // per slice and wave: 1 + the tile position of the wave's last key that is
  // not -inf (masked with -inf, or past L), 0 if there is none; the keys past
  // the largest add nothing to dQ or dpair
  __shared__ __attribute__((aligned(16))) int slive[2][4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int L = a.L, H = a.H, N = a.N;
  const int itiles = (L + kRows - 1) / kRows;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int it = rest % itiles;
  rest /= itiles;
  // rows longer than one key tile: with SPLIT each workgroup takes one key
  // tile and leaves an fp32 partial of dQ, summed over the tiles by bwd_fin
  // (the dpair block of a key tile stays in registers over the slices).
  // Without a pair bias there is no dpair to keep: one workgroup walks every
  // key tile of each slice in turn (KLOOP) and dQ stays in registers.
  constexpr bool KLOOP = !SPLIT && !HAS_PAIR;
  const int jtiles = SPLIT ? (L + TL::CH - 1) / TL::CH : 1;
  const int jt = SPLIT ? rest % jtiles : 0;
  if constexpr (SPLIT) rest /= jtiles;
  const int kjt = KLOOP ? (L + TL::CH - 1) / TL::CH : 1;  // key tiles walked per slice
  const int kc0 = jt * TL::CH;
  const int lk = L - kc0;  // keys of the row from this tile on (the first step's tile with KLOOP)
  const int ng = rest % a.n_groups_q;
  const int b = rest / a.n_groups_q;
  const int i = it * kRows + wave * 16 + col;
  const bool i_valid = i < L;
  const int ic = min(i, L - 1);
  const int n_begin = a.q_n0 + ng * a.Gq, n_end = min(a.q_n0 + a.q_nc, n_begin + a.Gq);
  const int ntiles = n_end - n_begin;
  const float scale = a.scale, c1 = a.scale * kLog2e;

  // resident pair bias: block blk, lane gets pair[ic][kc0 + 16 blk + 4 g + 0..3],
  // which is also the B operand of the 16x16x16 product that adds it (bf16)
  constexpr bool kPairMfma = HAS_PAIR && std::is_same<T, BF16>::value;
  u32x2 pbias[HAS_PAIR ? NB : 1];
  if constexpr (HAS_PAIR) {
    const uint16_t* prow = a.pair + (((size_t)b * H + h) * L + ic) * L;
    const bool pvec = (L % 4) == 0;
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      const int j = kc0 + 16 * blk + 4 * g;
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
  // A operands of the bias product: the parts of sqrt(D) on the diagonal,
  // lane (key row col, group g) holding A[col][4 g + e]
  constexpr int kSqP = kPairMfma ? kSqrtParts<D> : 1;
  short4_t sqid[kSqP];
  if constexpr (kPairMfma) {
    uint16_t sq[2];
    sqrt_d_parts<T>(a.sqrt_d, sq);
#pragma unroll
    for (int u = 0; u < kSqP; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) sqid[u][e] = (4 * g + e == col) ? (short)sq[u] : (short)0;
  }
  // bf16: the n-sum of dpair adds the fp32 dS (the bf16-rounded dS, 2^-9
  // relative, summed over N slices reaches the gradient tolerance where a
  // row's probability sits on few keys); fp16 rounds 8x finer and keeps the
  // identity MFMA
  constexpr bool kDpairF32 = std::is_same<T, BF16>::value;
  // identity A operand of the 16x16x16 dpair MFMA: lane (row col, group g) holds A[col][4g + e]
  short4_t ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (4 * g + e == col) ? T::one() : (short)0;

  TileCopy<D, NT> coff;
  tile_chunk_offsets<D, NT>(coff, kc0, L, a.sL, h, wave, lane);

  short8_t qop[KS32], gop[KS32], qnx[KS32], gnx[KS32], onx[KS32];
  float lse_nx = 0.f;
  uint32_t mraw = 0;
  const bool mask_thread = tid < TL::CH;
  auto load_rows = [&](int n) {  // Q, dO, O rows and the lse of slice n
    const int64_t row = b * a.sB + n * a.sN + ic * a.sL + h * D;  // element offset of the lane's row
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int d0 = 32 * s + 8 * g;
      short8_t qv = {0, 0, 0, 0, 0, 0, 0, 0}, gv = qv, ov = qv;
      if (d0 + 8 <= D) {
        qv = *reinterpret_cast<const short8_t*>(a.q + row + d0);
        gv = *reinterpret_cast<const short8_t*>(a.dout + row + d0);
        ov = *reinterpret_cast<const short8_t*>(a.out + row + d0);
      }
      qnx[s] = qv;
      gnx[s] = gv;
      onx[s] = ov;
    }
    lse_nx = a.lse[(((size_t)b * N + n) * H + h) * L + ic];
  };
  // the mask row of slice n for the key tile from key kt0 on
  auto load_mask = [&](int n, int kt0) {
    if (mask_thread) mraw = a.mask ? a.mask[((size_t)b * N + n) * L + min(kt0 + tid, L - 1)] : 0u;
  };
  // ltk: keys of the row from that tile on
  auto store_mask = [&](int buf, int ltk) {
    if (mask_thread) {  // whole waves: CH is a multiple of 64
      const float mv = (tid < ltk) ? T::to_f32((uint16_t)mraw) * a.sqrt_d : kNegInf;
      smk[buf][tid] = mv;
      const uint64_t live = __builtin_amdgcn_ballot_w64(mv != kNegInf);
      if (lane == 0) slive[buf][wave] = live ? 64 * wave + 64 - (int)__builtin_clzll(live) : 0;
    }
  };
  auto slice_ptr = [&](const uint16_t* base, int n) { return base + b * a.sB + n * a.sN; };

  floatx4 dpacc[WANT_DPAIR ? NB : 1];
#pragma unroll
  for (int blk = 0; blk < (WANT_DPAIR ? NB : 1); ++blk) dpacc[blk] = floatx4{0.f, 0.f, 0.f, 0.f};
  // the group's fp32 dpair partial of block blk (keys 16 blk + 4 g + 0..3 of query i)
  float* const dpdst = WANT_DPAIR ? a.dpair_part + ((((size_t)ng * a.B + b) * H + h) * L + ic) * L + kc0 : nullptr;
  if constexpr (WANT_DPAIR) {
    // a chunk after the first continues the sum its group slot holds (the
    // elements store_dpair writes; the others are never stored)
    if (a.dpair_carry && i_valid && ntiles > 0) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) {
        const int j = 16 * blk + 4 * g;
        if (j + 4 <= lk && (L % 4) == 0) {
          dpacc[blk] = *reinterpret_cast<const floatx4*>(dpdst + j);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (j + u < lk) dpacc[blk][u] = dpdst[j + u];
        }
      }
    }
  }
  auto store_dpair = [&](int blk) {
    if constexpr (WANT_DPAIR) {
      if (!i_valid) return;
      const int j = 16 * blk + 4 * g;
      if (j + 4 <= lk && (L % 4) == 0) {
        *reinterpret_cast<floatx4*>(dpdst + j) = dpacc[blk];
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j + u < lk) dpdst[j + u] = dpacc[blk][u];
      }
    }
  };

  // Q and dO rows of slice n into the operand registers, -lse log2e, and
  // delta = rowsum(dO * O) (written for bwd_kv3 by the first key tile's
  // workgroups) as the dP accumulator input -delta
  float nl = 0.f;
  floatx4 ndel = {0.f, 0.f, 0.f, 0.f};
  auto take_rows = [&](int n) {
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      qop[s] = qnx[s];
      gop[s] = gnx[s];
    }
    nl = (lse_nx == kNegInf) ? kNegInf : -lse_nx * kLog2e;  // rows with no finite score: P = 0
    // delta of this lane's query: dot over its 8 columns, then over the four
    // lane groups that hold the same query
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const u32x4 gw = __builtin_bit_cast(u32x4, gnx[s]), ow = __builtin_bit_cast(u32x4, onx[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) part = T::dot2(gw[e], ow[e], part);
    }
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (g == 0 && i_valid && jt == 0) a.delta[(((size_t)b * N + n) * H + h) * L + i] = part;
    ndel = floatx4{-part, -part, -part, -part};
  };

  if (ntiles > 0) {
    load_rows(n_begin);
    load_mask(n_begin, kc0);
    issue_tile<D, NT>(smem, slice_ptr(a.k, n_begin), slice_ptr(a.v, n_begin), coff, wave);
    store_mask(0, lk);
    vm_wait_all();
    take_rows(n_begin);
  }
  // the bias loads' -inf clamp once they and the first tile's copies are in
  // (a clamp next to its load would wait for each load in turn, and one
  // before the copies would hold the copies back; measured within the noise
  // at (1,512,256,8,8) and (1,768,768,4,32) against the clamps before them)
  if constexpr (kPairMfma) {
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      pbias[blk][0] = bf16x2_no_neg_inf(pbias[blk][0]);
      pbias[blk][1] = bf16x2_no_neg_inf(pbias[blk][1]);
    }
  }
  // The next slice's copies and row loads are completed before this slice's
  // dQ stores are issued.  With SPLIT (one key tile of a longer row per
  // workgroup, fp32 dQ partials) the next slice's rows are also taken then and
  // the barrier waits for LDS only, so nothing waits for the stores; rows of
  // one key tile measured faster with the plain barrier and the rows taken
  // after it (A/B on one device: bwd_q3 -4% at L = 256, +10% with SPLIT at
  // L = 768), and issue a slice's dQ stores after the next slice's barrier,
  // so that its wait for all memory operations does not wait for them
  // (bwd_q3 -2.7% at (1,256,256,4,32)).
  // Steps: (slice, key tile) pairs, the key tiles of a slice in turn (one per
  // slice unless KLOOP); dQ accumulates over a slice's key tiles.
  const int nsteps = ntiles * kjt;
  floatx4 dq[MB];
  // dQ = scale * dQ^T of slice n (after its last key tile): lane holds
  // d = 16 mb + 4 g + 0..3 of query i
  auto store_dq = [&](int n) {
    if (!i_valid) return;
    // dense row index of the fp32 partials (slices of the chunk)
    const size_t row = (((size_t)b * a.q_nc + (n - a.q_n0)) * L + i) * H + h;
    const int64_t qoff = b * a.sB + n * a.sN + i * a.sL + h * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int d = 16 * mb + 4 * g;
      if (d < D) {
        if constexpr (SPLIT) {
          float* dst = a.dq_part + ((size_t)jt * a.B * a.q_nc * L * H + row) * D + d;
          *reinterpret_cast<floatx4*>(dst) = dq[mb] * scale;
        } else {
          u32x2 w;
          w[0] = T::pack2(dq[mb][0] * scale, dq[mb][1] * scale);
          w[1] = T::pack2(dq[mb][2] * scale, dq[mb][3] * scale);
          *reinterpret_cast<u32x2*>(a.dq + qoff + d) = w;
        }
      }
    }
  };
  for (int t = 0; t < nsteps; ++t) {
    const int n = n_begin + t / kjt;
    const int jts = t % kjt;  // the step's key tile (0 unless KLOOP)
    const int lks = lk - jts * TL::CH;
    const int t1 = t + 1, jt1 = t1 % kjt;  // the next step
    const int n1 = n_begin + t1 / kjt;
    if constexpr (SPLIT) {
      lds_barrier();
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t > 0 && jts == 0) {
        store_dq(n - 1);  // the previous slice's (its dq registers are cleared below)
        take_rows(n);
      }
    }
    if (t1 < nsteps) {
      if constexpr (KLOOP) {
        if (kjt > 1) tile_chunk_offsets<D, NT>(coff, jt1 * TL::CH, L, a.sL, h, wave, lane);
      }
      issue_tile<D, NT>(smem + (t1 & 1) * TL::BUF_BYTES, slice_ptr(a.k, n1), slice_ptr(a.v, n1), coff, wave);
      if (jt1 == 0) load_rows(n1);
      load_mask(n1, kc0 + jt1 * TL::CH);
    }
    const uint8_t* kb = smem + (t & 1) * TL::BUF_BYTES;
    const uint8_t* vb = kb + TL::KCH * 16;
    const float* mkb = &smk[t & 1][4 * g];
    // keys of the slice up to the tile's last key that is not -inf
    int lkl;
    {
      const u32x4 lv = *reinterpret_cast<const u32x4*>(&slive[t & 1][0]);
      const int le = TL::CH > 128 ? max(max((int)lv[0], (int)lv[1]), max((int)lv[2], (int)lv[3]))
                                  : max((int)lv[0], (int)lv[1]);
      lkl = min(lks, __builtin_amdgcn_readfirstlane(le));
    }
    // Row (key) 16 blk + col of a tile: the swizzle depends on col only, so a
    // block's operands sit at a fixed offset from the lane's base address.
    // For D < 32 the k-slots past D read finite tile data that meets zeros in
    // the Q and dO operands.
    uint32_t kaddr[KS32], vaddr[KS32];
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int c = 4 * s + g;
      kaddr[s] = lds_addr(kb + (col * KC + ((c < KC ? c : 0) ^ kv_swz<KC>(col))) * 16);
      vaddr[s] = lds_addr(vb + (col * VC + ((c < VC ? c : 0) ^ kv_swz<VC>(col))) * 16);
    }
    const uint32_t maddr = lds_addr(mkb);
    // transposed K^T reads: row 4g + col/4 (+32 per step, +16 for the upper
    // half), column 16 mb + 4 (col % 4); the swizzle again depends on the lane only
    uint32_t ktaddr[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ktaddr[mb] = lds_addr(kb) + tr_off<KC>(4 * g + (col >> 2), 16 * mb + 4 * (col & 3));

    // Operands of one 32-key step (blocks 2 st and 2 st + 1): K rows, V rows
    // and the mask term, read one step ahead of the products that use them
    // (the reads complete under a step of vector work).
    struct StepOps {
      u32x4 k[2][KS32], v[2][KS32], m[2];
    };
    auto load_ops = [&](auto stc, StepOps& o) {
      constexpr int st = decltype(stc)::value;
      static_for<0, 2>([&](auto hc) {
        constexpr int hb = decltype(hc)::value, blk = 2 * st + hb;
        static_for<0, KS32>([&](auto sc_) {
          constexpr int s = decltype(sc_)::value;
          o.k[hb][s] = lds_b128_imm<blk * 16 * KC * 16>(kaddr[s]);
          o.v[hb][s] = lds_b128_imm<blk * 16 * VC * 16>(vaddr[s]);
        });
        o.m[hb] = lds_b128_imm<blk * 64>(maddr);
      });
    };
    auto touch_ops = [&](StepOps& o) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int s = 0; s < KS32; ++s) {
          reg_touch(o.k[hb][s]);
          reg_touch(o.v[hb][s]);
        }
        reg_touch(o.m[hb]);
      }
    };
    // S^T = K Q^T + sqrt(D) mask (+ sqrt(D) pair, bf16) and dP^T = V dO^T - delta of step st
    auto products = [&](auto stc, const StepOps& o, floatx4(&sv)[2], floatx4(&dv)[2]) {
      constexpr int st = decltype(stc)::value;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        floatx4 acc = __builtin_bit_cast(floatx4, o.m[hb]), accd = ndel;
#pragma unroll
        for (int s = 0; s < KS32; ++s) {
          acc = T::mfma16(__builtin_bit_cast(short8_t, o.k[hb][s]), qop[s], acc);
          accd = T::mfma16(__builtin_bit_cast(short8_t, o.v[hb][s]), gop[s], accd);
        }
        if constexpr (kPairMfma) {
          mfma_acc_handoff(acc);
#pragma unroll
          for (int u = 0; u < kSqP; ++u) acc = T::mfma16k16(sqid[u], __builtin_bit_cast(short4_t, pbias[2 * st + hb]), acc);
        }
        sv[hb] = acc;
        dv[hb] = accd;
      }
    };

    if (jts == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) dq[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    floatx4 sc[2][2], dp[2][2];
    StepOps ops;
    load_ops(std::integral_constant<int, 0>{}, ops);
    lgkm_wait<0>();
    touch_ops(ops);
    products(std::integral_constant<int, 0>{}, ops, sc[0], dp[0]);
    if constexpr (NSTEP > 1) load_ops(std::integral_constant<int, 1>{}, ops);
    static_for<0, NSTEP>([&](auto stc) {
      constexpr int st = decltype(stc)::value;
      constexpr int cur = st & 1;
      // The next step's products are issued before this step's vector work
      // (their operands were read during the previous step), and the
      // operands of the step after are read.  Rows past L read finite tile
      // data and are never used.
      if constexpr (st + 1 < NSTEP) {
        lgkm_wait<0>();
        touch_ops(ops);
        products(std::integral_constant<int, st + 1>{}, ops, sc[cur ^ 1], dp[cur ^ 1]);
        if constexpr (st + 2 < NSTEP) load_ops(std::integral_constant<int, st + 2>{}, ops);
      }
      if (32 * st < lkl) {
        short4_t kt[2 * MB];  // [mb][lo/hi 16 keys]
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          kt[2 * mb] = lds_tr_imm<st * 32 * KC * 16>(ktaddr[mb]);
          kt[2 * mb + 1] = lds_tr_imm<st * 32 * KC * 16 + 16 * KC * 16>(ktaddr[mb]);
        }
        // keep the vector work below the reads so that it covers their latency
        __builtin_amdgcn_sched_barrier(0);
        float ds[2][4];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int blk = 2 * st + hb;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x;
            if constexpr (HAS_PAIR && !kPairMfma) {
              const uint32_t w = pbias[blk][r / 2];
              const float sv = (r & 1) ? T::fma_mix_hi(sc[cur][hb][r], scale, w) : T::fma_mix_lo(sc[cur][hb][r], scale, w);
              x = __builtin_fmaf(sv, kLog2e, nl);
            } else {
              x = __builtin_fmaf(sc[cur][hb][r], c1, nl);
            }
            ds[hb][r] = __builtin_amdgcn_exp2f(x) * dp[cur][hb][r];
          }
        }
        const u32x4 dw = {T::pack2(ds[0][0], ds[0][1]), T::pack2(ds[0][2], ds[0][3]), T::pack2(ds[1][0], ds[1][1]),
                          T::pack2(ds[1][2], ds[1][3])};
        const short8_t dsb = __builtin_bit_cast(short8_t, dw);
        if constexpr (WANT_DPAIR) {
          if constexpr (kDpairF32) {
            // accumulator register r of the identity product is the lane's own
            // operand element r, so the n-sum is an fp32 add in place
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
              for (int r = 0; r < 4; ++r) dpacc[2 * st + hb][r] += ds[hb][r];
          } else {
            dpacc[2 * st] = T::mfma16k16(ident, __builtin_bit_cast(short4_t, u32x2{dw[0], dw[1]}), dpacc[2 * st]);
            dpacc[2 * st + 1] = T::mfma16k16(ident, __builtin_bit_cast(short4_t, u32x2{dw[2], dw[3]}), dpacc[2 * st + 1]);
          }
        }
        // the transposed and prefetch reads complete here, after the vector
        // work (the packed dS is an operand of the wait)
        short8_t dsw = dsb;
        lgkm_wait_after(dsw);
#pragma unroll
        for (int k = 0; k < 2 * MB; ++k) reg_touch(kt[k]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dq[mb] = T::mfma16(cat4(kt[2 * mb], kt[2 * mb + 1]), dsw, dq[mb]);
      }
      // rows longer than one key tile: blocks 2 st and 2 st + 1 of the dpair
      // slot are final after the group's last step reaches them, and their
      // stores go out under the remaining steps instead of all at the end
      // (A/B on MI355X: bwd_q3 -8% at (1,768,768,4,32); rows of one key tile
      // measured the same or slower, and store at the end)
      if constexpr (WANT_DPAIR && SPLIT) {
        if (t == nsteps - 1) {
          store_dpair(2 * st);
          store_dpair(2 * st + 1);
        }
      }
    });
    vm_wait_all();  // the next step's copies and loads
    if (t1 < nsteps) {
      store_mask(t1 & 1, lk - jt1 * TL::CH);  // its buffer was last read during step t-1
      if constexpr (SPLIT) take_rows(n + 1);
    }
    // SPLIT: the slice's dQ partial now (the next step's barrier waits for
    // LDS only); otherwise after the next step's barrier, which waits for
    // all memory operations and would otherwise wait for these stores
    if constexpr (SPLIT) {
      if (jts == kjt - 1) store_dq(n);
    }
  }
  if constexpr (!SPLIT) {
    if (nsteps > 0) store_dq(n_begin + (nsteps - 1) / kjt);  // the last slice's
  }

  if constexpr (WANT_DPAIR && !SPLIT) {
    if (ntiles > 0) {
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) store_dpair(blk);
    }
  }
}

// ---------------------------------------------------------------- bwd_kv3
//
// The mirror image: wave w owns keys 16w..16w+15 of the workgroup's 16 NW (lane
// = key, S layout with query rows); K and V rows of the lane's key are the
// MFMA B operands; per n the Q and dO rows of the slice arrive in LDS
// (same tile layout), -lse log2e and -delta per query through LDS.  Per
// 32-query step:
//   S  = Q K^T + sqrt(D) mask_j          (lane constant as accumulator input)
//   dP = dO V^T - delta_i                (accumulator input read from LDS)
//   P = exp2(...),  dS = P dP
//   dV^T += dO^T P,  dK^T += Q^T dS      (dO^T, Q^T by transposed LDS reads)
//   dmask partial += column sums of dS   (MFMA against a row of ones)
// The pair-bias columns of the workgroup's keys come through an LDS slab of
// their own, split by wave (each wave's 16 columns), read with transposed
// reads.  Rows that fit one query tile: read once per workgroup, their copy
// beside the first Q and dO tile, and kept in registers for the whole n-group.
// Longer rows (MULTI): per n the queries come in tiles of CH; dK, dV and dmask
// accumulate over the tiles, and each (n, tile)'s columns are copied while the
// previous tile is computed, each wave refilling its region as soon as it has
// read it.
template <class T, int D, bool HAS_PAIR, bool WANT_DMASK, bool MULTI, int NW>
__global__ __launch_bounds__(64 * NW) void evo_bwd_kv3_kernel(BwdArgs a) {
  using TL = KVTile<D>;
  constexpr int KS32 = (D + 31) / 32;
  constexpr int NB = TL::CH / 16;  // 16-query blocks per tile
  constexpr int NSTEP = TL::CH / 32;
  constexpr int MB = (D + 15) / 16;
  constexpr int KC = TL::KC, VC = TL::VC;
  constexpr int NT = 64 * NW, kRows = 16 * NW;
  constexpr int kSlab = HAS_PAIR ? TL::CH * kRows * 2 : 0;  // pair[CH queries][the workgroup's keys]
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * TL::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sslab[HAS_PAIR ? kSlab : 16];
  __shared__ __attribute__((aligned(16))) float slse[2][TL::CH];  // -lse log2e; -inf past L / no finite score
  __shared__ __attribute__((aligned(16))) float sndel[2][TL::CH]; // -delta

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int L = a.L, H = a.H, N = a.N;
  const int jtiles = (L + kRows - 1) / kRows;
  const int ngroups = a.n_groups_k;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int h = wg % H;
  int rest = wg / H;
  const int jt = rest % jtiles;
  rest /= jtiles;
  const int ng = rest % ngroups;
  const int b = rest / ngroups;
  const int j = jt * kRows + wave * 16 + col;  // this lane's key
  const bool j_valid = j < L;
  const int jc = min(j, L - 1);
  const int n_begin = ng * a.Gk, n_end = min(N, n_begin + a.Gk);
  const int ntiles = n_end - n_begin;
  const int qtiles = MULTI ? (L + TL::CH - 1) / TL::CH : 1;  // query tiles per slice
  const int nu = ntiles * qtiles;                             // (n, query tile) steps
  const float scale = a.scale, c1 = a.scale * kLog2e;
  const uint16_t* pbase = HAS_PAIR ? a.pair + ((size_t)b * H + h) * L * L : nullptr;
  const int kc0k = jt * kRows;  // the workgroup's first key

  // bias block qb of a query tile: lane gets pair[q0 + 16 qb + 4 g + r][j], r = 0..3
  u32x2 pbias[HAS_PAIR ? NB : 1];
  // The bias columns of a query tile (L % 8 == 0) come through an LDS slab
  // split by wave, each wave's region holding only its own 16 columns (CH rows
  // of 32 bytes, contiguous), so a wave reads its region as soon as its own
  // copies are done, and (rows longer than one query tile) refills it as soon
  // as it has read it, with no workgroup barrier; the regions' 32-byte rows
  // keep a transposed read's four rows on different banks.  The slab has LDS
  // of its own, so its first copy goes out with the first Q and dO tile.
  auto issue_slab_w = [&](int q0) {
    uint8_t* dst = sslab + wave * (TL::CH * 32);
#pragma unroll
    for (int i = 0; i < TL::CH * 2 / 64; ++i) {
      const int c = 64 * i + lane;  // 16-byte chunk c: row c / 2, keys 8 (c % 2) ..
      const uint16_t* src =
          pbase + (size_t)min(q0 + (c >> 1), L - 1) * L + min(kc0k + 16 * wave + 8 * (c & 1), L - 8);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + 64 * 16 * i), 16, 0, 0);
    }
  };
  // the wave's region into pbias (reads the compiler does not track, so it
  // does not wait for the copies in flight; the wait below completes them)
  auto read_slab_w = [&]() {
    const uint8_t* src = sslab + wave * (TL::CH * 32);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int row = 16 * qb + 4 * g + (col >> 2);
      pbias[qb] = __builtin_bit_cast(u32x2, lds_read_tr_asm(src, (row * 16 + 4 * (col & 3)) * 2));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) asm volatile("" : "+v"(pbias[qb]));
  };
  auto gather_bias = [&](int q0) {  // L % 8 != 0: column reads straight from memory
    const uint16_t* prow = pbase + jc;
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      uint32_t t4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) t4[r] = prow[(size_t)min(q0 + 16 * qb + 4 * g + r, L - 1) * L];
      pbias[qb][0] = t4[0] | (t4[1] << 16);
      pbias[qb][1] = t4[2] | (t4[3] << 16);
    }
  };

  // ---- resident pair bias (one query tile), rows of odd length (the slab's
  // are read after the prologue's copies)
  if constexpr (HAS_PAIR && !MULTI) {
    if ((L % 8) != 0) gather_bias(0);
  }

  // ones in row 0 of the column-sum operand
  short8_t ones = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = T::one();
  }

  TileCopy<D, NT> coff;
  tile_chunk_offsets<D, NT>(coff, 0, L, a.sL, h, wave, lane);

  // ---- per-slice key operands (B of S = Q K^T and dP = dO V^T): lane = key
  short8_t kop[KS32], vop[KS32], knx[KS32], vnx[KS32];
  uint32_t mnx = 0;
  float lse_nx = 0.f, del_nx = 0.f;
  const bool row_thread = tid < TL::CH;
  auto load_keys = [&](int n) {  // K, V rows and the mask of the lane's key
    const int64_t row = b * a.sB + n * a.sN + jc * a.sL + h * D;
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int d0 = 32 * s + 8 * g;
      short8_t kv = {0, 0, 0, 0, 0, 0, 0, 0}, vv = kv;
      if (d0 + 8 <= D) {
        kv = *reinterpret_cast<const short8_t*>(a.k + row + d0);
        vv = *reinterpret_cast<const short8_t*>(a.v + row + d0);
      }
      knx[s] = kv;
      vnx[s] = vv;
    }
    mnx = a.mask ? a.mask[((size_t)b * N + n) * L + jc] : 0u;
  };
  auto slice_ptr = [&](const uint16_t* base, int n) { return base + b * a.sB + n * a.sN; };
  int q0_nx = 0;
  auto load_rows = [&](int n, int q0) {  // lse, delta of query q0 + tid
    q0_nx = q0;
    if (row_thread) {
      const size_t ri = (((size_t)b * N + n) * H + h) * L + min(q0 + tid, L - 1);
      lse_nx = a.lse[ri];
      del_nx = a.delta[ri];
    }
  };
  auto store_rows = [&](int buf) {
    if (row_thread) {
      // queries past L, or with no finite score, get P = 0
      slse[buf][tid] = (q0_nx + tid < L && lse_nx != kNegInf) ? -lse_nx * kLog2e : kNegInf;
      sndel[buf][tid] = -del_nx;
    }
  };
  // the asynchronous copy of step u's Q and dO tile into buffer buf
  auto issue_qo = [&](int u, int buf) {
    const int n = n_begin + u / qtiles, q0 = (u % qtiles) * TL::CH;
    const uint16_t* qs = slice_ptr(a.q, n);
    const uint16_t* os = slice_ptr(a.dout, n);
    uint8_t* dst = smem + buf * TL::BUF_BYTES;
    if constexpr (MULTI) {
      TileCopy<D, NT> tc;
      tile_chunk_offsets<D, NT>(tc, q0, L, a.sL, h, wave, lane);
      issue_tile<D, NT>(dst, qs, os, tc, wave);
    } else {
      issue_tile<D, NT>(dst, qs, os, coff, wave);
    }
  };

  floatx4 mk4 = {0.f, 0.f, 0.f, 0.f};
  bool kdead = false;  // every key of this wave is -inf in the current slice: dK = dV = dmask = 0
  // the slice's K and V rows of the lane's key into the operand registers, and
  // sqrt(D) * mask of the key as the score accumulator input
  auto take_keys = [&]() {
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      kop[s] = knx[s];
      vop[s] = vnx[s];
    }
    const float mk = j_valid ? T::to_f32((uint16_t)mnx) * a.sqrt_d : kNegInf;
    mk4 = floatx4{mk, mk, mk, mk};
    kdead = __builtin_amdgcn_ballot_w64(mk == kNegInf) == ~0ull;
  };
  floatx4 dk[MB], dv[MB], dmk = {0.f, 0.f, 0.f, 0.f};
  // bf16: the dmask column sums add the fp32 dS (a bf16-rounded dS, 2^-9
  // relative, summed over H x L terms reaches the gradient tolerance when a
  // row's probability sits on few keys); fp16 rounds 8x finer and keeps the
  // column-sum MFMA
  constexpr bool kDmaskF32 = std::is_same<T, BF16>::value;
  float dmsum = 0.f;
  if (nu > 0) {
    load_keys(n_begin);
    load_rows(n_begin, 0);
    issue_qo(0, 0);
    if constexpr (HAS_PAIR) {
      if ((L % 8) == 0) issue_slab_w(0);
    }
    store_rows(0);
    vm_wait_all();
    take_keys();
    if constexpr (HAS_PAIR && !MULTI) {
      if ((L % 8) == 0) read_slab_w();  // its own copies are done
    }
  }
  // The next step's copies and loads are completed, and its rows and keys
  // taken, before this step's dK, dV stores are issued: no wait (a barrier's
  // or the compiler's) then waits for those stores.
  for (int u = 0; u < nu; ++u) {
    const int t = u / qtiles, qt = u % qtiles, q0 = qt * TL::CH;
    const int n = n_begin + t;
    const int lq = L - q0;  // queries of the row from this tile on
    lds_barrier();
    if (qt == 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        dk[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
        dv[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      dmk = floatx4{0.f, 0.f, 0.f, 0.f};
      dmsum = 0.f;
    }
    if constexpr (MULTI && HAS_PAIR) {
      // this tile's bias columns; the wave's region is then free for the next tile's
      if ((L % 8) == 0) {
        read_slab_w();
      } else {
        gather_bias(q0);
      }
    }
    if (u + 1 < nu) {
      const int n1 = n_begin + (u + 1) / qtiles, qt1 = (u + 1) % qtiles;
      issue_qo(u + 1, (u + 1) & 1);
      if constexpr (MULTI && HAS_PAIR) {
        if ((L % 8) == 0) issue_slab_w(qt1 * TL::CH);
      }
      load_rows(n1, qt1 * TL::CH);
      if (qt1 == 0) load_keys(n1);
    }
    const uint8_t* qb_ = smem + (u & 1) * TL::BUF_BYTES;
    const uint8_t* ob_ = qb_ + TL::KCH * 16;
    // per-lane LDS byte addresses (see bwd_q3)
    uint32_t qaddr[KS32], oaddr[KS32];
#pragma unroll
    for (int s = 0; s < KS32; ++s) {
      const int c = 4 * s + g;
      qaddr[s] = lds_addr(qb_ + (col * KC + ((c < KC ? c : 0) ^ kv_swz<KC>(col))) * 16);
      oaddr[s] = lds_addr(ob_ + (col * VC + ((c < VC ? c : 0) ^ kv_swz<VC>(col))) * 16);
    }
    const uint32_t laddr = lds_addr(&slse[u & 1][4 * g]), daddr = lds_addr(&sndel[u & 1][4 * g]);
    uint32_t qtaddr[MB], otaddr[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      qtaddr[mb] = lds_addr(qb_) + tr_off<KC>(4 * g + (col >> 2), 16 * mb + 4 * (col & 3));
      otaddr[mb] = lds_addr(ob_) + tr_off<VC>(4 * g + (col >> 2), 16 * mb + 4 * (col & 3));
    }

    // Operands of one 32-query step (blocks 2 st, 2 st + 1): Q rows, dO rows,
    // -delta and -lse log2e of the block's queries, read one step ahead of
    // the products.  -lse log2e is consumed by the vector work a step later,
    // so it rotates through three slots.
    struct StepOps {
      u32x4 q[2][KS32], o[2][KS32], d[2];
    };
    u32x4 nlr[3][2];
    auto load_ops = [&](auto stc, StepOps& o) {
      constexpr int st = decltype(stc)::value;
      static_for<0, 2>([&](auto hc) {
        constexpr int hb = decltype(hc)::value, blk = 2 * st + hb;
        static_for<0, KS32>([&](auto sc_) {
          constexpr int s = decltype(sc_)::value;
          o.q[hb][s] = lds_b128_imm<blk * 16 * KC * 16>(qaddr[s]);
          o.o[hb][s] = lds_b128_imm<blk * 16 * VC * 16>(oaddr[s]);
        });
        o.d[hb] = lds_b128_imm<blk * 64>(daddr);
        nlr[st % 3][hb] = lds_b128_imm<blk * 64>(laddr);
      });
    };
    auto touch_ops = [&](StepOps& o, int slot) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
        for (int s = 0; s < KS32; ++s) {
          reg_touch(o.q[hb][s]);
          reg_touch(o.o[hb][s]);
        }
        reg_touch(o.d[hb]);
      }
      // slot is a compile-time constant at every call
      if (slot == 0) { reg_touch(nlr[0][0]); reg_touch(nlr[0][1]); }
      if (slot == 1) { reg_touch(nlr[1][0]); reg_touch(nlr[1][1]); }
      if (slot == 2) { reg_touch(nlr[2][0]); reg_touch(nlr[2][1]); }
    };
    // S = Q K^T + sqrt(D) mask_j and dP = dO V^T - delta_i of one step
    auto products = [&](const StepOps& o, floatx4(&sv)[2], floatx4(&dv)[2]) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        floatx4 acc = mk4, accd = __builtin_bit_cast(floatx4, o.d[hb]);
#pragma unroll
        for (int s = 0; s < KS32; ++s) {
          acc = T::mfma16(__builtin_bit_cast(short8_t, o.q[hb][s]), kop[s], acc);
          accd = T::mfma16(__builtin_bit_cast(short8_t, o.o[hb][s]), vop[s], accd);
        }
        sv[hb] = acc;
        dv[hb] = accd;
      }
    };

    if (!kdead) {
      floatx4 sc[2][2], dp[2][2];
      StepOps ops;
      load_ops(std::integral_constant<int, 0>{}, ops);
      lgkm_wait<0>();
      touch_ops(ops, 0);
      products(ops, sc[0], dp[0]);
      if constexpr (NSTEP > 1) load_ops(std::integral_constant<int, 1>{}, ops);
      static_for<0, NSTEP>([&](auto stc) {
        constexpr int st = decltype(stc)::value;
        constexpr int cur = st & 1;
        if constexpr (st + 1 < NSTEP) {
          lgkm_wait<0>();
          touch_ops(ops, (st + 1) % 3);
          products(ops, sc[cur ^ 1], dp[cur ^ 1]);
          if constexpr (st + 2 < NSTEP) load_ops(std::integral_constant<int, st + 2>{}, ops);
        }
        if (32 * st < lq) {
          short4_t tt[4 * MB];  // [mb][q lo, q hi, o lo, o hi]
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            tt[4 * mb + 0] = lds_tr_imm<st * 32 * KC * 16>(qtaddr[mb]);
            tt[4 * mb + 1] = lds_tr_imm<st * 32 * KC * 16 + 16 * KC * 16>(qtaddr[mb]);
            tt[4 * mb + 2] = lds_tr_imm<st * 32 * VC * 16>(otaddr[mb]);
            tt[4 * mb + 3] = lds_tr_imm<st * 32 * VC * 16 + 16 * VC * 16>(otaddr[mb]);
          }
          // keep the vector work below the reads so that it covers their latency
          __builtin_amdgcn_sched_barrier(0);
          float pv[2][4], ds[2][4];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const int blk = 2 * st + hb;
            const floatx4 nl4 = __builtin_bit_cast(floatx4, nlr[st % 3][hb]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x;
              if constexpr (HAS_PAIR) {
                const uint32_t w = pbias[blk][r / 2];
                const float sv = (r & 1) ? T::fma_mix_hi(sc[cur][hb][r], scale, w) : T::fma_mix_lo(sc[cur][hb][r], scale, w);
                x = __builtin_fmaf(sv, kLog2e, nl4[r]);
              } else {
                x = __builtin_fmaf(sc[cur][hb][r], c1, nl4[r]);
              }
              const float p = __builtin_amdgcn_exp2f(x);
              pv[hb][r] = p;
              ds[hb][r] = p * dp[cur][hb][r];
            }
          }
          const short8_t pb = __builtin_bit_cast(
              short8_t, u32x4{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]), T::pack2(pv[1][0], pv[1][1]),
                              T::pack2(pv[1][2], pv[1][3])});
          const short8_t db = __builtin_bit_cast(
              short8_t, u32x4{T::pack2(ds[0][0], ds[0][1]), T::pack2(ds[0][2], ds[0][3]), T::pack2(ds[1][0], ds[1][1]),
                              T::pack2(ds[1][2], ds[1][3])});
          if constexpr (WANT_DMASK) {
            if constexpr (kDmaskF32) {
              dmsum += ((ds[0][0] + ds[0][1]) + (ds[0][2] + ds[0][3])) + ((ds[1][0] + ds[1][1]) + (ds[1][2] + ds[1][3]));
            } else {
              dmk = T::mfma16(ones, db, dmk);
            }
          }
          // the transposed and prefetch reads complete here, after the vector
          // work (the packed P and dS are operands of the wait)
          short8_t pbw = pb, dbw = db;
          lgkm_wait_after(pbw, dbw);
#pragma unroll
          for (int k = 0; k < 4 * MB; ++k) reg_touch(tt[k]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            dk[mb] = T::mfma16(cat4(tt[4 * mb], tt[4 * mb + 1]), dbw, dk[mb]);
            dv[mb] = T::mfma16(cat4(tt[4 * mb + 2], tt[4 * mb + 3]), pbw, dv[mb]);
          }
        }
      });
    }  // !kdead
    vm_wait_all();  // the next step's copies and loads
    if (u + 1 < nu) {
      store_rows((u + 1) & 1);  // its buffers were last read during step u-1
      if ((u + 1) % qtiles == 0) take_keys();
    }
    // ---- dK = scale * dK^T, dV: lane holds d = 16 mb + 4 g + 0..3 of key j
    if constexpr (WANT_DMASK && kDmaskF32) {
      if (qt == qtiles - 1) {  // the four lane groups holding key j hold its partial sums
        dmsum += __shfl_xor(dmsum, 16);
        dmsum += __shfl_xor(dmsum, 32);
        dmk[0] = dmsum;
      }
    }
    if (j_valid && qt == qtiles - 1) {
      const int64_t row = b * a.sB + n * a.sN + j * a.sL + h * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int d = 16 * mb + 4 * g;
        if (d < D) {
          u32x2 wk, wv;
          wk[0] = T::pack2(dk[mb][0] * scale, dk[mb][1] * scale);
          wk[1] = T::pack2(dk[mb][2] * scale, dk[mb][3] * scale);
          wv[0] = T::pack2(dv[mb][0], dv[mb][1]);
          wv[1] = T::pack2(dv[mb][2], dv[mb][3]);
          *reinterpret_cast<u32x2*>(a.dk + row + d) = wk;
          *reinterpret_cast<u32x2*>(a.dv + row + d) = wv;
        }
      }
      if (WANT_DMASK && g == 0) a.dmask_part[(((size_t)b * N + n) * H + h) * L + j] = dmk[0];
    }
  }
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HP>
static hipError_t launch_tile_t(const BwdArgs& a, hipStream_t st) {
  const bool want_dmask = a.dmask != nullptr;
  const bool want_dpair = a.dpair != nullptr;
  // bwd_q3 forms delta and leaves it in the workspace for bwd_kv3
  constexpr int NW = kWaves, kRows = 16 * kWaves;
  const int gridq = a.B * a.H * ((a.L + kRows - 1) / kRows) * a.n_groups_q;
  prof_begin(K_BWD_Q, st);
  if (want_dpair)
    hipLaunchKernelGGL((evo_bwd_q3_kernel<T, D, HP, true, false, NW>), dim3(gridq), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((evo_bwd_q3_kernel<T, D, HP, false, false, NW>), dim3(gridq), dim3(64 * NW), 0, st, a);
  prof_end(K_BWD_Q, st);
  const int gridk = a.B * a.H * ((a.L + kRows - 1) / kRows) * a.n_groups_k;
  prof_begin(K_BWD_KV, st);
  if (want_dmask)
    hipLaunchKernelGGL((evo_bwd_kv3_kernel<T, D, HP, true, false, NW>), dim3(gridk), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((evo_bwd_kv3_kernel<T, D, HP, false, false, NW>), dim3(gridk), dim3(64 * NW), 0, st, a);
  prof_end(K_BWD_KV, st);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_tile_d(const BwdArgs& a, hipStream_t st) {
  return a.pair ? launch_tile_t<T, D, true>(a, st) : launch_tile_t<T, D, false>(a, st);
}

template <class T>
static hipError_t launch_tile_dt(const BwdArgs& a, int D, hipStream_t st) {
  switch (D) {
    case 8: return launch_tile_d<T, 8>(a, st);
    case 16: return launch_tile_d<T, 16>(a, st);
    case 32: return launch_tile_d<T, 32>(a, st);
    case 64: return launch_tile_d<T, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(const BwdArgs& a, int D, bool bf16, hipStream_t stream) {
  return bf16 ? launch_tile_dt<BF16>(a, D, stream) : launch_tile_dt<F16>(a, D, stream);
}

template <class T, int D, bool HP>
static hipError_t launch_split_t(const BwdArgs& a, int part, hipStream_t st) {
  constexpr int NW = kWaves, kRows = 16 * kWaves;
  if (part == 0) {
    // bwd_q3 over the chunk's slices and every key tile
    const int jtiles = (a.L + KVTile<D>::CH - 1) / KVTile<D>::CH;
    const int grid = a.B * a.H * ((a.L + kRows - 1) / kRows) * jtiles * a.n_groups_q;
    prof_begin(K_BWD_Q, st);
    if (a.dpair)
      hipLaunchKernelGGL((evo_bwd_q3_kernel<T, D, HP, true, true, NW>), dim3(grid), dim3(64 * NW), 0, st, a);
    else
      hipLaunchKernelGGL((evo_bwd_q3_kernel<T, D, HP, false, true, NW>), dim3(grid), dim3(64 * NW), 0, st, a);
    prof_end(K_BWD_Q, st);
  } else if (part == 2) {
    // no pair bias: bwd_q3 with every key tile of a slice in one workgroup
    if constexpr (!HP) {
      const int grid = a.B * a.H * ((a.L + kRows - 1) / kRows) * a.n_groups_q;
      prof_begin(K_BWD_Q, st);
      hipLaunchKernelGGL((evo_bwd_q3_kernel<T, D, false, false, false, NW>), dim3(grid), dim3(64 * NW), 0, st, a);
      prof_end(K_BWD_Q, st);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    // key side over query tiles; it reads the delta bwd_q3 wrote
    const int gridk = a.B * a.H * ((a.L + kRows - 1) / kRows) * a.n_groups_k;
    prof_begin(K_BWD_KV, st);
    if (a.dmask)
      hipLaunchKernelGGL((evo_bwd_kv3_kernel<T, D, HP, true, true, NW>), dim3(gridk), dim3(64 * NW), 0, st, a);
    else
      hipLaunchKernelGGL((evo_bwd_kv3_kernel<T, D, HP, false, true, NW>), dim3(gridk), dim3(64 * NW), 0, st, a);
    prof_end(K_BWD_KV, st);
  }
  return hipGetLastError();
}

template <class T>
static hipError_t launch_split_dt(const BwdArgs& a, int D, int part, hipStream_t st) {
  const bool hp = a.pair != nullptr;
  switch (D) {
    case 8: return hp ? launch_split_t<T, 8, true>(a, part, st) : launch_split_t<T, 8, false>(a, part, st);
    case 16: return hp ? launch_split_t<T, 16, true>(a, part, st) : launch_split_t<T, 16, false>(a, part, st);
    case 32: return hp ? launch_split_t<T, 32, true>(a, part, st) : launch_split_t<T, 32, false>(a, part, st);
    case 64: return hp ? launch_split_t<T, 64, true>(a, part, st) : launch_split_t<T, 64, false>(a, part, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_q_split(const BwdArgs& a, int D, bool bf16, int part, hipStream_t stream) {
  return bf16 ? launch_split_dt<BF16>(a, D, part, stream) : launch_split_dt<F16>(a, D, part, stream);
}

}  // namespace evo
