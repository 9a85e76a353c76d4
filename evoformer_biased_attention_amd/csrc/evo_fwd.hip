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
//   slices; otherwise each block's values are loaded from L2 seven blocks
//   ahead (three at D = 64) into a ring of registers.
//   The mask bias is the QK^T product's accumulator input: per tile an fp32
//   row of sqrt(D)*mask[j] (-inf for keys past L) sits in LDS, and each block
//   starts its S^T accumulator from it, so the scale turns it back into
//   mask[j] at no VALU or extra MFMA cost.
//   Keys masked with -inf add nothing to a row (P = 0 there).  Per tile the
//   end of its last key that is not -inf is recorded, and the 32-key blocks
//   past it (the padding at the end of a row) are not computed.
//   Running max: the exponent base is only moved when a row's block max
//   exceeds it by more than 8 (log2 units), so exp values stay below 2^8 and
//   the accumulator is rarely rescaled.
#include "evo_common.h"
#include "evo_kernels.h"
#include "evo_prof.h"

namespace evo {

constexpr int kFwdWaves = 4;
constexpr int kFwdRows = 32 * kFwdWaves;  // query rows per workgroup
constexpr float kTau2 = 8.f;  // the exponent base may lag the row max by up to 8 (log2 units)
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFastSum = 256.f;  // 2^8: a block sum below it keeps the exponent base (no block max)

// Key tiles of the forward without a pair bias at D <= 32: 128 keys (256 at
// D = 8, where a row is 16 bytes), half the LDS of the shared tile, so that
// three 4-wave workgroups (three waves per SIMD, at most 168 VGPRs each) share
// a CU (measured on MI355X: -13% at (1,384,512,8,32)).  With a pair bias the
// resident bias registers do not fit that budget, nor does D = 64: those keep
// the shared tile at two waves per SIMD.
template <int D>
struct FwdTileNoPair {
  static constexpr int CH = (D == 8) ? 256 : 128;
  static constexpr int KC = D / 8;
  static constexpr int VC = (D < 32 ? 32 : D) / 8;
  static constexpr int KCH = CH * KC;
  static constexpr int VCH = CH * VC;
  static constexpr int TCH = KCH + VCH;
  static constexpr int BUF_BYTES = TCH * 16;
  static_assert(TCH % 256 == 0, "tile must split evenly over 256 threads");
};
template <int D, bool HAS_PAIR>
constexpr bool kFwdThreeWaves = !HAS_PAIR && D <= 32;
template <int D, bool HAS_PAIR>
using FwdTile = typename std::conditional<kFwdThreeWaves<D, HAS_PAIR>, FwdTileNoPair<D>, KVTile<D>>::type;

template <int D>
struct FwdShape {
  static constexpr int KSTEPS_D = (D + 15) / 16;  // 16-wide k-steps over d (zero past D)
  static constexpr int MB = (D + 31) / 32;        // 32-row blocks of O^T
};

// Pair-bias values of one 32-key block, 16 per lane (query i, half), in one of
// two orders.  kMfma: the B operand of the bias product, which adds the bias
// to the S^T accumulator through the MFMA (an identity over the block's keys,
// scaled by sqrt(D) as the mask term is, times the pair rows): position
// 8 s + e holds pair[i][j0 + 16 s + 8 half + e].  Otherwise the S^T accumulator
// order, for a bias added to the scores by the VALU: position 4 q + u holds
// pair[i][j0 + 8 q + 4 half + u].  vec: L is a multiple of the run of
// consecutive keys (8 or 4), so the runs are aligned vector loads.
// kSettle: columns >= L read zero and the MFMA order (that of bf16) takes its
// -inf values out (bf16x2_no_neg_inf), which makes the caller wait for the
// loads at once.  Without it the loaded values are left as they arrive, for
// a caller that applies pair_no_neg_inf before the product: columns >= L then
// hold finite values of the row's last keys, which the mask term turns into
// -inf scores as it does for zeros.
template <bool kMfma, bool kSettle = true>
__device__ __forceinline__ void load_pair_ops(short8_t (&dst)[2], const uint16_t* prow, int j0, int L, int half,
                                              bool vec) {
  constexpr int G = kMfma ? 8 : 4;  // consecutive keys per run
  uint32_t w[8];
#pragma unroll
  for (int g = 0; g < 16 / G; ++g) {
    const int j = j0 + (kMfma ? 16 * g + 8 * half : 8 * g + 4 * half);
    if (vec) {  // uniform; j + G - 1 < L whenever j < L
      if constexpr (kMfma) {
        u32x4 v = *reinterpret_cast<const u32x4*>(prow + min(j, L - G));
        if (kSettle && j >= L) v = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * g + e] = v[e];
      } else {
        u32x2 v = *reinterpret_cast<const u32x2*>(prow + min(j, L - G));
        if (kSettle && j >= L) v = u32x2{0u, 0u};
        w[2 * g] = v[0];
        w[2 * g + 1] = v[1];
      }
    } else {
      uint32_t t[G];
#pragma unroll
      for (int e = 0; e < G; ++e) t[e] = (!kSettle || j + e < L) ? (uint32_t)prow[min(j + e, L - 1)] : 0u;
#pragma unroll
      for (int e = 0; e < G; e += 2) w[(g * G + e) / 2] = t[e] | (t[e + 1] << 16);
    }
  }
  if constexpr (kMfma && kSettle) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = bf16x2_no_neg_inf(w[e]);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) dst[s] = __builtin_bit_cast(short8_t, u32x4{w[4 * s], w[4 * s + 1], w[4 * s + 2], w[4 * s + 3]});
}

// The -inf values of pair-bias operands in the MFMA order taken out in place
// (the second half of load_pair_ops' settling, for operands loaded without it).
__device__ __forceinline__ void pair_no_neg_inf(short8_t (&p)[2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    u32x4 w = __builtin_bit_cast(u32x4, p[s]);
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = bf16x2_no_neg_inf(w[e]);
    p[s] = __builtin_bit_cast(short8_t, w);
  }
}

template <class T, int D, bool HAS_MASK, bool HAS_PAIR, int RES>
__global__ __launch_bounds__(256, (kFwdThreeWaves<D, HAS_PAIR> ? 3 : 2)) void evo_fwd_kernel(FwdArgs a) {
  using S = FwdShape<D>;
  using TL = FwdTile<D, HAS_PAIR>;
  constexpr int kMcBufs = (std::is_same<T, F16>::value && D <= 32) ? 2 : 1;
  // two K/V tile buffers; with a resident pair bias the same bytes first hold
  // the workgroup's 128 x (32 RES) bias slab
  constexpr int kSlab = RES > 0 ? kFwdRows * RES * 64 : 0;
  constexpr int kSmem = 2 * TL::BUF_BYTES > kSlab ? 2 * TL::BUF_BYTES : kSlab;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  __shared__ __attribute__((aligned(16))) float smk[2][TL::CH];  // sqrt(D) * mask per key, -inf past L
  // per tile and wave: 1 + the tile position of the wave's last key that is
  // not -inf (masked with -inf, or past L), 0 if there is none
  __shared__ __attribute__((aligned(16))) int slive[2][4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // known uniform to the compiler
  const int half = lane >> 5;
  const int L = a.L, H = a.H, N = a.N;

  // workgroup -> (h, i-tile, n-group, b) with h fastest: the ids one XCD gets
  // are consecutive, so all heads and query tiles of a run of slices share
  // that XCD's L2 (the heads of a row are interleaved in memory)
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  int h, it, ng, b;
  if constexpr (RES == 0 && HAS_PAIR) {
    // a streamed pair bias (rows longer than one key tile) is re-read for
    // every slice: (two heads, query tile, n-group) order instead, so that
    // the workgroups one XCD runs at a time read the bias planes of two
    // heads, which stay in its L2 (two heads share the cache lines of a Q,
    // K, V row; measured on MI355X at (1,768,768,4,32): forward -6% against
    // the order below, whose XCDs each read all heads' planes)
    const int hp = (H % 2) == 0 ? 2 : 1;
    int r = wg;
    const int hl = r % hp;
    r /= hp;
    it = r % a.i_tiles;
    r /= a.i_tiles;
    ng = r % a.n_groups;
    r /= a.n_groups;
    h = (r % (H / hp)) * hp + hl;
    b = r / (H / hp);
  } else {
    h = wg % H;
    int rest = wg / H;
    it = rest % a.i_tiles;
    rest /= a.i_tiles;
    ng = rest % a.n_groups;
    b = rest / a.n_groups;
  }
  if (a.balance) {
    // (b, n-group) by balanced_unit_rank over the batch entries ranked by the
    // live 32-key blocks of their slice 0, a block counted when its first key
    // is not -inf (padding at the end of a row: the blocks the kernel
    // computes); ties keep the order of b.  One load per lane (entry, block),
    // one ballot; every wave takes the same decision on its own.
    const int nb = (L + 31) / 32;  // a.B * nb <= 64 (checked by the launcher)
    bool live = false;
    if (lane < a.B * nb) live = a.mask[(size_t)(lane / nb) * N * L + (lane % nb) * 32] != T::kNegInfBits;
    const uint64_t bits = __builtin_amdgcn_ballot_w64(live);
    const uint64_t seg = nb >= 64 ? ~0ull : ((1ull << nb) - 1);
    const int unit = H * a.i_tiles;
    const int r = balanced_unit_rank(wg, (int)gridDim.x / 8, unit, a.B * a.n_groups);
    const int want = r / a.n_groups;  // rank of the batch entry among all
    int cost[kBalanceMaxB];
#pragma unroll
    for (int bb = 0; bb < kBalanceMaxB; ++bb) {
      const uint64_t m = bb < a.B ? (bits >> (bb * nb)) & seg : 0ull;
      cost[bb] = bb < a.B ? (m ? 64 - (int)__builtin_clzll(m) : 0) : -1;
    }
    int pick = 0;
#pragma unroll
    for (int bb = 0; bb < kBalanceMaxB; ++bb) {
      int rank = 0;
#pragma unroll
      for (int o = 0; o < kBalanceMaxB; ++o) rank += (cost[o] > cost[bb] || (cost[o] == cost[bb] && o < bb)) ? 1 : 0;
      if (bb < a.B && rank == want) pick = bb;
    }
    b = pick;
    ng = r % a.n_groups;
  }

  const int i = it * kFwdRows + wave * 32 + (lane & 31);
  const bool i_valid = i < L;
  const int ic = min(i, L - 1);  // rows past L compute a copy of row L-1 and are not stored
  const int n_begin = ng * a.G;
  const int n_end = min(N, n_begin + a.G);
  const int nchunks = (L + TL::CH - 1) / TL::CH;
  const int ntiles = (n_end - n_begin) * nchunks;

  // ---- pair-bias values (held for the whole kernel when the row fits one tile).
  // bf16 adds them through the MFMA (no mixed-precision FMA takes a bf16
  // operand, so the VALU would first widen each value); fp16 adds them in the
  // VALU (one mixed-precision FMA per score costs less than the extra MFMAs).
  constexpr bool kPairMfma = HAS_PAIR && std::is_same<T, BF16>::value;
  short8_t pres[RES > 0 ? RES : 1][2];
  const uint16_t* prow = nullptr;
  const bool pvec = (L % (kPairMfma ? 8 : 4)) == 0;
  if constexpr (HAS_PAIR) {
    prow = a.pair + (((size_t)b * H + h) * L + ic) * L;
    if constexpr (RES > 0) {
      if ((L % 8) == 0) {
        // Coalesced: the workgroup's 128 rows x L pair-bias slab goes to LDS by
        // asynchronous 16-byte copies (chunk c of row r stored at position
        // c ^ (r & 15), so the per-lane reads below are spread over the banks),
        // then every lane picks its values.  Runs before the first K/V tile.
        constexpr int RC = RES * 4;  // 16-byte chunks per staged row
        const int row0 = it * kFwdRows;
        // uniform base (the slab's first row) plus a 32-bit offset per chunk
        const char* pbase = reinterpret_cast<const char*>(a.pair + (((size_t)b * H + h) * L + row0) * L);
        const int rlim = L - 1 - row0;
#pragma unroll
        for (int k = 0; k < kFwdRows * RC / 256; ++k) {
          const int base = wave_u * 64 + 256 * k;
          const int q = base + lane;
          const int r = q / RC, pos = q % RC;
          const int c = min(pos ^ (r & 15), L / 8 - 1);
          const uint32_t off = ((uint32_t)min(r, rlim) * (uint32_t)L + 8u * (uint32_t)c) * 2u;
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(pbase + off),
                                           (__attribute__((address_space(3))) void*)(smem + base * 16), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int r = wave * 32 + (lane & 31);
#pragma unroll
        for (int kb = 0; kb < RES; ++kb)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            if constexpr (kPairMfma) {
              const int c = 4 * kb + 2 * s2 + half;  // chunk holding keys 32 kb + 16 s2 + 8 half .. +7
              u32x4 v = *reinterpret_cast<const u32x4*>(smem + (r * RC + ((c ^ (r & 15)) % RC)) * 16);
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = bf16x2_no_neg_inf(v[e]);
              pres[kb][s2] = __builtin_bit_cast(short8_t, v);
            } else {
              // keys 32 kb + 8 q + 4 half .. +3 for q = 2 s2, 2 s2 + 1: the
              // half-chunk at byte 8 half of chunk 4 kb + q
              const int c0 = 4 * kb + 2 * s2, c1 = c0 + 1;
              const u32x2 v0 = *reinterpret_cast<const u32x2*>(smem + (r * RC + ((c0 ^ (r & 15)) % RC)) * 16 + 8 * half);
              const u32x2 v1 = *reinterpret_cast<const u32x2*>(smem + (r * RC + ((c1 ^ (r & 15)) % RC)) * 16 + 8 * half);
              pres[kb][s2] = __builtin_bit_cast(short8_t, u32x4{v0[0], v0[1], v1[0], v1[1]});
            }
          }
        __syncthreads();  // the slab area is reused by the K/V tiles
      } else {
        // all loads first, then the -inf clamp (keys past L: the mask term,
        // always present when L is not a multiple of 32, makes them -inf)
#pragma unroll
        for (int kb = 0; kb < RES; ++kb) load_pair_ops<kPairMfma, false>(pres[kb], prow, kb * 32, L, half, pvec);
        if constexpr (kPairMfma) {
#pragma unroll
          for (int kb = 0; kb < RES; ++kb) pair_no_neg_inf(pres[kb]);
        }
      }
    }
  }

  // A operands of the bias product (bf16): the parts of sqrt(D) on the
  // diagonal of the block's keys, so the product adds sqrt(D) pair[i][j] to
  // S^T[j][i] as the mask term adds sqrt(D) mask[j]; for k-step s, lane
  // (key m, half) holds it at position m - 16 s - 8 half when that lies in 0..7
  constexpr int kSqParts = kSqrtParts<D>;
  short8_t pid[kPairMfma ? kSqParts : 1][2];
  if constexpr (kPairMfma) {
    uint16_t sq[2];
    sqrt_d_parts<T>(a.sqrt_d, sq);
    const int m = lane & 31;
#pragma unroll
    for (int u = 0; u < kSqParts; ++u)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pid[u][s2][e] = (m == 16 * s2 + 8 * half + e) ? (short)sq[u] : (short)0;
  }
  // scale to log2 units of an accumulator that holds every term of the score
  const float c1 = a.scale * kLog2e;

  short8_t qop[S::KSTEPS_D], qnext[S::KSTEPS_D];
  uint32_t mraw = 0;  // this thread's mask value for the next tile (thread < CH)

  auto load_q = [&](short8_t (&dst)[S::KSTEPS_D], int n) {
    const uint16_t* qrow = a.q + b * a.sB + n * a.sN + ic * a.sL + h * D;
#pragma unroll
    for (int s = 0; s < S::KSTEPS_D; ++s) {
      const int c = 16 * s + 8 * half;
      short8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (c + 8 <= D) v = *reinterpret_cast<const short8_t*>(qrow + c);
      dst[s] = v;
    }
  };
  // The mask row of a tile: thread tid loads key kc0 + tid (clamped), and
  // after the tile's blocks it stores sqrt(D) * mask, or -inf for keys past L.
  // HAS_MASK also covers rows whose length is not a multiple of 32 without a
  // user mask: the mask is then zero and only the tail is -inf, so no
  // per-score tail test is needed anywhere.
  auto load_mask = [&](int n, int kc0) {
    if constexpr (HAS_MASK) {
      if (tid < TL::CH) mraw = a.mask ? a.mask[((size_t)b * N + n) * L + min(kc0 + tid, L - 1)] : 0u;
    }
  };
  auto store_mask = [&](int buf, int kc0) {
    if constexpr (HAS_MASK) {
      if (tid < TL::CH) {  // whole waves: CH is a multiple of 64
        const float mv = (kc0 + tid < L) ? T::to_f32((uint16_t)mraw) * a.sqrt_d : kNegInf;
        smk[buf][tid] = mv;
        const uint64_t live = __builtin_amdgcn_ballot_w64(mv != kNegInf);
        if (lane == 0) slive[buf][wave] = live ? 64 * wave + 64 - (int)__builtin_clzll(live) : 0;
      }
    }
  };
  // issue the asynchronous copy of tile t into LDS buffer (t & 1): a uniform
  // base pointer (the tile's first key row of the slice) plus a 32-bit byte
  // offset per 16-byte chunk (K-layout chunks, then V-layout chunks; rows past
  // L clamp to L - 1), so the copies address by scalar base + vector offset.
  // A thread's copy blocks of 64 chunks start on multiples of 64 chunks, so
  // with C chunks per row (C divides 64) a lane's row within its block is
  // lane / C, its chunk lane % C, and its row's swizzle (period 16 rows; the
  // blocks' first rows differ by multiples of 16) the same in every block of a
  // kind: each copy adds only its block's first row, a wave-uniform offset.
  constexpr int NCH = TL::TCH / 256;  // chunks per thread
  static_assert(TL::KCH % 256 == 0, "K chunks must fill whole copy rounds");
  static_assert(64 % TL::KC == 0 && 64 % TL::VC == 0, "a copy block must hold whole rows");
  const uint32_t sl2 = (uint32_t)a.sL * 2u, hd2 = (uint32_t)(h * D) * 2u;
  auto issue_tile = [&](int t) {
    const int c = t % nchunks;
    const int n = n_begin + t / nchunks;
    const int lim = min(TL::CH - 1, L - 1 - c * TL::CH);
    const int64_t row0 = b * a.sB + n * a.sN + (int64_t)(c * TL::CH) * a.sL;
    const char* kbase = reinterpret_cast<const char*>(a.k + row0);
    const char* vbase = reinterpret_cast<const char*>(a.v + row0);
    uint8_t* buf = smem + (t & 1) * TL::BUF_BYTES;
    const bool full = lim == TL::CH - 1;  // no row of the tile lies past L
    // the two per-lane offsets are recomputed per tile (a dozen integer ops)
    // rather than kept in registers across the tile loop
    uint32_t ln = (uint32_t)lane;  // unsigned: the divisions below are shifts
    asm volatile("" : "+v"(ln));
    uint32_t kv_lane[2];  // per-lane byte offset within a copy block: K, V
    {
      const int rk = (int)(ln / TL::KC), rv = (int)(ln / TL::VC);
      const int ck = (int)(ln % TL::KC) ^ kv_swz<TL::KC>(wave_u * 64 / TL::KC + rk);
      int cv = (int)(ln % TL::VC) ^ kv_swz<TL::VC>(wave_u * 64 / TL::VC + rv);
      if (cv >= D / 8) cv = 0;  // columns the transposed reads touch but never use
      kv_lane[0] = (uint32_t)rk * sl2 + hd2 + 16u * (uint32_t)ck;
      kv_lane[1] = (uint32_t)rv * sl2 + hd2 + 16u * (uint32_t)cv;
    }
    constexpr int kRounds = TL::KCH / 256;  // K chunks fill the first rounds
    auto copy = [&](auto full_c) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const bool is_k = i < kRounds;
        const int base = wave_u * 64 + 256 * i;  // wave-uniform
        const int rb = is_k ? base / TL::KC : (base - TL::KCH) / TL::VC;  // block's first row
        uint32_t off;
        if constexpr (decltype(full_c)::value) {
          off = (uint32_t)rb * sl2 + kv_lane[is_k ? 0 : 1];
        } else {
          const int lrow = (int)(is_k ? ln / TL::KC : ln / TL::VC);
          const uint32_t lcol = kv_lane[is_k ? 0 : 1] - (uint32_t)lrow * sl2;
          off = (uint32_t)min(rb + lrow, lim) * sl2 + lcol;
        }
        const char* src = (is_k ? kbase : vbase) + off;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (__attribute__((address_space(3))) void*)(buf + base * 16), 16, 0, 0);
      }
    };
    if (full) {
      copy(std::true_type{});
    } else {
      copy(std::false_type{});
    }
  };

  // A resident pair bias means rows of one key tile: every tile is a whole
  // slice, whose first block's PV product takes a zero accumulator input in
  // place of a cleared O^T accumulator.
  constexpr bool kOneChunk = RES > 0;
  floatx16 oacc[S::MB];
#pragma unroll
  for (int mb2 = 0; mb2 < S::MB; ++mb2) oacc[mb2] = floatx16{};
  // m_used: the row's exponent base in log2 units; the row sum in two chains
  float m_used = kNegInf, l_part = 0.f, l_part2 = 0.f;

  // Per-lane byte offsets within a tile buffer.  The swizzle repeats every 16
  // rows, so block jb of a tile adds the constant 32 jb rows, which goes into
  // the read instruction's offset field.
  uint32_t koff[S::KSTEPS_D];
#pragma unroll
  for (int s = 0; s < S::KSTEPS_D; ++s) {
    const int r = lane & 31, c = 2 * s + half;
    koff[s] = (c < TL::KC) ? (uint32_t)((r * TL::KC + (c ^ kv_swz<TL::KC>(r))) * 16) : 0u;
  }
  uint32_t voff[S::MB][2];  // V^T reads of rows 4 g + i16 / 4 and 8 rows further
  {
    const int qg = lane >> 4, i16 = lane & 15, g = qg >> 1;
    const int row = 4 * g + (i16 >> 2);
#pragma unroll
    for (int mb2 = 0; mb2 < S::MB; ++mb2) {
      const int col = 16 * (qg & 1) + 32 * mb2 + 4 * (i16 & 3);
      voff[mb2][0] = (uint32_t)(TL::KCH * 16 + tr_off<TL::VC>(row, col));
      voff[mb2][1] = (uint32_t)(TL::KCH * 16 + tr_off<TL::VC>(row + 8, col));
    }
  }

  // ---- K operands of one 32-key block (asm reads, completed by the next PV wait)
  auto k_fetch = [&](auto jbc, const uint32_t bufa, short8_t (&kop)[S::KSTEPS_D]) {
    constexpr int jb = decltype(jbc)::value;
    static_for<0, S::KSTEPS_D>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if (2 * s + half < TL::KC) {
        kop[s] = __builtin_bit_cast(short8_t, lds_b128_imm<jb * 32 * TL::KC * 16>(bufa + koff[s]));
      } else {
        kop[s] = short8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    });
  };
  // ---- mask term of one 32-key block in the S^T accumulator layout: lane
  // (query, half) register r holds key 8 (r / 4) + 4 half + r % 4.  Ordinary
  // (compiler-visible) loads: the values become an MFMA accumulator input, and
  // the compiler must see these writes to keep them clear of the MFMAs still
  // reading the previous block's input from the same registers.
  auto mc_fetch = [&](int buf, const int jb, floatx16& dst) {
    if constexpr (HAS_MASK) {
      const float* row = &smk[buf][jb * 32 + 4 * half];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v = *reinterpret_cast<const floatx4*>(row + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * q + e] = v[e];
      }
    }
  };
  // The same, issued as reads the compiler does not track (it otherwise waits
  // for every LDS read in flight, the K prefetch included, before them); used
  // for the prefetch two blocks ahead and completed by the wait before the PV
  // product.  maddr is the LDS address of smk[buf][4 half].
  auto mc_fetch_async = [&](auto jbc, const uint32_t maddr, floatx16& dst) {
    if constexpr (HAS_MASK) {
      constexpr int jb = decltype(jbc)::value;
      static_for<0, 4>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        const floatx4 v = __builtin_bit_cast(floatx4, lds_b128_imm<(jb * 32 + 8 * q) * 4>(maddr));
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * q + e] = v[e];
      });
    }
  };
  // ---- S^T block = K Q^T + sqrt(D) mask + sqrt(D) pair for 32 keys
  auto qk_block = [&](const short8_t (&kop_in)[S::KSTEPS_D], const floatx16& minit,
                      const short8_t (&pq)[2]) -> floatx16 {
    floatx16 acc = HAS_MASK ? minit : floatx16{};
#pragma unroll
    for (int s = 0; s < S::KSTEPS_D; ++s) acc = T::mfma(kop_in[s], qop[s], acc);
    if constexpr (kPairMfma) {
#pragma unroll
      for (int u = 0; u < kSqParts; ++u) {
        acc = T::mfma(pid[u][0], pq[0], acc);
        acc = T::mfma(pid[u][1], pq[1], acc);
      }
    }
    return acc;
  };

  // ---- bias, online softmax and O^T += V^T P^T for one block whose scores are in acc
  auto softmax_pv = [&](const floatx16& acc, const int tb, auto jbc, const short8_t (&pb)[2],
                        short8_t (&kpre)[S::KSTEPS_D], floatx16& mpre, auto prec, const bool pre_live) {
    constexpr int jb = decltype(jbc)::value, jb_pre = decltype(prec)::value;
    const uint32_t bufa = lds_addr(smem + tb * TL::BUF_BYTES);
    // V^T operands first: the reads complete under the softmax VALU work
    // K operands and the mask term two blocks ahead, completed by the wait below
    if constexpr (jb_pre >= 0) {
      if (pre_live) {
        k_fetch(prec, bufa, kpre);
        if constexpr (kMcBufs == 2) {
          mc_fetch_async(prec, lds_addr(&smk[tb][4 * half]), mpre);
        } else {
          mc_fetch(tb, jb_pre, mpre);
        }
      }
    }
    short4_t vt[4 * S::MB];  // [t][mb][lo/hi]
    static_for<0, 2>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      static_for<0, S::MB>([&](auto mc_) {
        constexpr int mb2 = decltype(mc_)::value;
        constexpr int off = (jb * 32 + 16 * t) * TL::VC * 16;
        vt[(t * S::MB + mb2) * 2 + 0] = lds_tr_imm<off>(bufa + voff[mb2][0]);
        vt[(t * S::MB + mb2) * 2 + 1] = lds_tr_imm<off>(bufa + voff[mb2][1]);
      });
    });
    // the scores in log2 units are sc * cf
    float sc[16];
    float cf = c1;
    if constexpr (HAS_PAIR && !kPairMfma) {
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const uint32_t w = __builtin_bit_cast(u32x4, pb[rr / 8])[(rr % 8) / 2];
        sc[rr] = T::fma_mix_lo(acc[rr], a.scale, w);
        sc[rr + 1] = T::fma_mix_hi(acc[rr + 1], a.scale, w);
      }
      cf = kLog2e;
    } else {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sc[rr] = acc[rr];
    }
    uint32_t pk[8];
    // The exponent base moves only when it has to: it may lag the row max by up
    // to 8 (log2 units), so exp values stay below 2^8.
    // The exps are first taken against the current base m_used: if a row's
    // block sum stays below 2^8 in both halves, each of its probabilities
    // does, so no score lies more than 8 (log2 units) above the base and the
    // max-first rule would keep the base too: the row's block is done
    // without its maximum.  Otherwise (or on the first block of a row, whose
    // base is still -inf) the block max is formed and the row's base moved to
    // it when it exceeds the old one by more than 8 (log2 units), rescaling
    // the O^T accumulator and the row sums, and the exps are taken again.
    // Both rules give the same base and the same sums (up to the rounding of
    // the comparison itself), so a row's result does not depend on the rule
    // its block took.
    float bs0, bs1;  // block sums, two chains
    auto exps = [&](const float neg_ml) {
      bs0 = 0.f;
      bs1 = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rr], cf, neg_ml));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[rr + 1], cf, neg_ml));
        pk[rr / 2] = T::pack2(p0, p1);
        // fp16: the rounded pair by v_dot2; bf16 sums the fp32 values
        if ((rr / 2) & 1) {
          bs1 = T::rowsum_add(bs1, p0, p1, pk[rr / 2]);
        } else {
          bs0 = T::rowsum_add(bs0, p0, p1, pk[rr / 2]);
        }
      }
    };
    // The choice is made per query row (the lane and its partner half), so a
    // row's bits never depend on the other rows of the wave.
    const bool first = m_used == kNegInf;
    bool redo = first;
    if (__builtin_amdgcn_ballot_w64(!first) != 0) {
      exps(first ? 0.f : -m_used);
      redo = first || !(bs0 + bs1 < kFastSum);
    }
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      {  // the row redoes when either half of it does
        float fa = redo ? 1.f : 0.f, fb = fa;
        xhalf_swap(fa, fb);
        redo = (fa + fb) > 0.f;
      }
      // block max in two chains of three-input maxima.  Written as assembly:
      // the scores come out of the MFMA or of assembly (v_fma_mix_f32), so
      // the compiler would first canonicalize them for its own maximum;
      // scores are never NaN for finite inputs.
      auto max3 = [](float x, float y, float z) {
        float r;
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
        return r;
      };
      float mb0 = max3(sc[0], sc[1], sc[2]), mb1 = max3(sc[8], sc[9], sc[10]);
      mb0 = max3(mb0, sc[3], sc[4]);
      mb1 = max3(mb1, sc[11], sc[12]);
      mb0 = max3(mb0, sc[5], sc[6]);
      mb1 = max3(mb1, sc[13], sc[14]);
      mb0 = max3(mb0, mb1, sc[7]);
      float mb = max3(mb0, sc[15], sc[15]);
      {  // with the partner half (lane ^ 32) holding the same query row
        float xa = mb, xb = mb;
        xhalf_swap(xa, xb);
        mb = max3(xa, xb, xb) * cf;  // cf > 0: the max in log2 units
      }
      // rows that keep their base recompute the same exps
      const bool need = redo && mb > m_used + kTau2;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mb : m_used;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;
        m_used = m_new;
        l_part *= alpha;
        l_part2 *= alpha;
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) oacc[mb2][rr] *= alpha;
      }
      exps((m_used == kNegInf) ? 0.f : -m_used);
    }
    l_part += bs0;
    l_part2 += bs1;
    // the V^T and prefetch reads complete here, after the exps (the packed
    // probabilities are operands of the wait)
    u32x4 bop[2] = {u32x4{pk[0], pk[1], pk[2], pk[3]}, u32x4{pk[4], pk[5], pk[6], pk[7]}};
    lgkm_wait_after(bop[0], bop[1]);
#pragma unroll
    for (int k = 0; k < 4 * S::MB; ++k) reg_touch(vt[k]);
#pragma unroll
    for (int k = 0; k < S::KSTEPS_D; ++k) reg_touch(kpre[k]);
    if constexpr (kMcBufs == 2) reg_touch(mpre);
    // (a slice's first block: the first product starts from zero, and the
    // accumulator's earlier contents, rescaled by 0 above, are not read)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int mb2 = 0; mb2 < S::MB; ++mb2)
        oacc[mb2] = T::mfma(cat4(vt[(t * S::MB + mb2) * 2], vt[(t * S::MB + mb2) * 2 + 1]),
                            __builtin_bit_cast(short8_t, bop[t]),
                            (kOneChunk && jb == 0 && t == 0) ? floatx16{} : oacc[mb2]);
    }
  };

  // score accumulators and the mask terms of a tile's blocks (every block's are
  // written before they are read; cleared once, so they always hold values)
  floatx16 sacc[2], mcb[2] = {floatx16{}, floatx16{}};

  // Streamed pair bias (rows longer than one key tile): a ring of kRing
  // blocks' values, block j in slot j % kRing, each loaded kRing - 1 blocks
  // before the block that uses it (across tile boundaries: the pair bias
  // does not depend on n), so no load latency falls at the start of a tile;
  // the loads leave their values as they arrive (no wait at the load).
  // Measured on MI355X at (1,768,768,4,32), with the work order of a streamed
  // bias: forward 908 us loading each tile's bias at its top, 757 us with a
  // ring of 4, 728 us with 8 (803 with 2).
  constexpr bool kStream = RES == 0 && HAS_PAIR;
  constexpr int kRing = TL::CH / 32 >= 8 ? 8 : 4;  // a tile's blocks (it must divide them)
  short8_t pring[kStream ? kRing : 1][2];
  // the next tile's copies go out in the middle of a streamed tile, after the
  // bias loads of the blocks before it: waiting for those never waits for
  // the copies, which have half a tile to complete
  constexpr int kIssueAt = kStream ? TL::CH / 64 - 1 : 0;

  // ---- pipeline: tile t computes from buffer t&1 while tile t+1 streams into the other
  if (ntiles > 0) {
    if constexpr (kStream) {
#pragma unroll
      for (int j = 0; j < kRing - 1; ++j) load_pair_ops<kPairMfma, false>(pring[j], prow, j * 32, L, half, pvec);
    }
    issue_tile(0);
    load_mask(n_begin, 0);
    load_q(qnext, n_begin);
    store_mask(0, 0);
    vm_wait_all();
#pragma unroll
    for (int s = 0; s < S::KSTEPS_D; ++s) qop[s] = qnext[s];
  }
  // Tile t's copies (and its mask / Q loads) are completed by each thread
  // before tile t-1's output stores are issued, so the barrier at the top of
  // tile t waits for no store.
  for (int t = 0; t < ntiles; ++t) {
    const int n = n_begin + t / nchunks;
    const int c = t % nchunks;
    const int kc0 = c * TL::CH;
    lds_barrier();  // everyone's copies of tile t are done; everyone has finished tile t-1
    if (c == 0) {
      if constexpr (!kOneChunk) {
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2) oacc[mb2] = floatx16{};
      }
      m_used = kNegInf;
      l_part = 0.f;
      l_part2 = 0.f;
    }
    // the next tile's copies, mask row and Q rows
    auto issue_next = [&]() {
      if (t + 1 < ntiles) {
        issue_tile(t + 1);
        const int n1 = n_begin + (t + 1) / nchunks;
        load_mask(n1, ((t + 1) % nchunks) * TL::CH);
        if ((t + 1) % nchunks == 0) load_q(qnext, n1);
      }
    };
    if constexpr (!kStream) issue_next();
    const int kc0n = ((t + 1) % nchunks) * TL::CH;  // the next tile's first key
    const int tb = t & 1;
    const uint8_t* buf = smem + tb * TL::BUF_BYTES;
    // blocks of the tile, software-pipelined: while block jb is in its softmax,
    // the QK^T MFMAs of block jb+1 run and the K operands and mask term of
    // block jb+2 load
    // blocks up to the tile's last key that is not -inf
    int nblk = min(TL::CH, L - kc0 + 31) / 32;
    if constexpr (HAS_MASK) {
      const u32x4 lv = *reinterpret_cast<const u32x4*>(&slive[tb][0]);
      const int le = TL::CH > 128 ? max(max((int)lv[0], (int)lv[1]), max((int)lv[2], (int)lv[3]))
                                  : max((int)lv[0], (int)lv[1]);
      nblk = min(nblk, (__builtin_amdgcn_readfirstlane(le) + 31) / 32);
    }
    if constexpr (kOneChunk) {
      // a slice with no block to compute stores zeros from a cleared accumulator
      if (nblk == 0) {
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2) oacc[mb2] = floatx16{};
      }
    }
    {
      constexpr int NB = (RES > 0 && RES < TL::CH / 32) ? RES : TL::CH / 32;
      short8_t kreg[2][S::KSTEPS_D];
      // fp16 with D <= 32: the mask term of block j sits in mcb[j & 1], so the prefetch for
      // block j + 2 never writes the registers the QK^T product just issued for
      // block j + 1 still reads as its accumulator input, and it is issued
      // untracked (the compiler does not then wait for the K prefetch before
      // it: -3% at (1,256,256,4,32)).  bf16 and D = 64, whose kernels are at
      // the register limit: block 0 in mcb[0] and every later block in mcb[1],
      // loaded by tracked reads.
      auto msel = [](int j) { return kMcBufs == 2 ? (j & 1) : (j == 0 ? 0 : 1); };
      const uint32_t bufa = lds_addr(buf);
      k_fetch(std::integral_constant<int, 0>{}, bufa, kreg[0]);
      mc_fetch(tb, 0, mcb[0]);
      if (nblk > 1) {
        k_fetch(std::integral_constant<int, 1>{}, bufa, kreg[1]);
        mc_fetch(tb, 1, mcb[1]);
      }
      {
        short4_t none[2] = {};
        lds_wait_all(none, kreg[0]);
        lds_wait_all(none, kreg[1]);
      }
      // pair-bias values of block j (a dummy without a pair bias)
      auto pops = [&](auto jc) -> const short8_t(&)[2] {
        constexpr int j = decltype(jc)::value;
        if constexpr (RES > 0) {
          return pres[j < RES ? j : 0];
        } else {
          return pring[kStream ? j % kRing : 0];
        }
      };
      // streamed bf16 bias: a block's -inf values are taken out just before its
      // product, two blocks after its load (not at the load, which would wait
      // for it there)
      if constexpr (kStream && kPairMfma) pair_no_neg_inf(pring[0]);
      sacc[0] = qk_block(kreg[0], mcb[0], pops(std::integral_constant<int, 0>{}));
      static_for<0, NB>([&](auto jbc) {
        constexpr int jb = decltype(jbc)::value;
        if constexpr (kStream) {
          // block jb + kRing - 1 (of this tile or the next) into the slot
          // block jb - 1 has finished with; loaded also past the tile's last
          // live block, so that the next tile's first blocks are there
          constexpr int jl = jb + kRing - 1;
          if constexpr (jl < NB) {
            load_pair_ops<kPairMfma, false>(pring[jl % kRing], prow, kc0 + jl * 32, L, half, pvec);
          } else {
            if (t + 1 < ntiles)
              load_pair_ops<kPairMfma, false>(pring[jl % kRing], prow, kc0n + (jl - NB) * 32, L, half, pvec);
          }
          if constexpr (jb == kIssueAt) issue_next();
        }
        if (jb < nblk) {
          if constexpr (jb + 1 < NB) {
            if (jb + 1 < nblk) {
              if constexpr (kStream && kPairMfma) pair_no_neg_inf(pring[(jb + 1) % kRing]);
              sacc[(jb + 1) & 1] = qk_block(kreg[(jb + 1) & 1], mcb[msel(jb + 1)],
                                            pops(std::integral_constant<int, jb + 1>{}));
            }
          }
          // the K operands of block jb + 2 are read only when it exists
          const bool pre_live = jb + 2 < nblk;
          constexpr int jpre = jb + 2 < NB ? jb + 2 : -1;
          softmax_pv(sacc[jb & 1], tb, jbc, pops(jbc), kreg[jb & 1], mcb[msel(jb + 2)],
                     std::integral_constant<int, jpre>{}, pre_live);
        }
      });
    }
    // Tile t+1's copies and loads were issued a tile ago.  Its mask row and
    // Q rows are taken now, before this tile's output stores are issued, so
    // that no wait for them (the compiler's included) waits for those stores.
    vm_wait_all();
    if (t + 1 < ntiles) {
      store_mask((t + 1) & 1, ((t + 1) % nchunks) * TL::CH);  // its buffer was last read during tile t-1
      if ((t + 1) % nchunks == 0) {
#pragma unroll
        for (int s = 0; s < S::KSTEPS_D; ++s) qop[s] = qnext[s];
      }
    }
    if (c == nchunks - 1) {
      // ---- epilogue of slice n: normalise, store O and lse
      const float l_tot = xhalf_sum(l_part + l_part2);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      {
        // lanes l and l^32 hold alternating runs of 4 columns of the same row
        // (lane half h: columns 32 mb + 8 q + 4 h .. +3); each run is stored as
        // one 8-byte write, the two halves' runs side by side in memory
        uint16_t* orow = a.out + b * a.sB + n * a.sN + ic * a.sL + h * D;
#pragma unroll
        for (int mb2 = 0; mb2 < S::MB; ++mb2)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 w;
            w[0] = T::pack2(oacc[mb2][4 * q] * inv, oacc[mb2][4 * q + 1] * inv);
            w[1] = T::pack2(oacc[mb2][4 * q + 2] * inv, oacc[mb2][4 * q + 3] * inv);
            const int d = 32 * mb2 + 8 * q + 4 * half;
            if (i_valid && d < D) *reinterpret_cast<u32x2*>(orow + d) = w;
          }
        if (i_valid && half == 0 && a.lse != nullptr) {
          const float lse = (m_used == kNegInf || !(l_tot > 0.f)) ? kNegInf : __builtin_fmaf(m_used, kLn2, __logf(l_tot));
          a.lse[(((size_t)b * N + n) * H + h) * L + i] = lse;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch

template <class T, int D, bool HM, bool HP>
static hipError_t launch_fwd_t(const FwdArgs& a_in, hipStream_t stream) {
  FwdArgs a = a_in;
  const int grid = a.B * a.H * a.i_tiles * a.n_groups;
  // the balanced work order: a mask to rank the batch entries by (one wave's
  // lanes cover every entry's blocks), two workgroups per CU in one round (not
  // the three-wave tiles), units that split evenly over the XCDs' halves, and
  // not a streamed pair bias (which has an order of its own)
  a.balance = 0;
  const bool streamed = HP && a.L > KVTile<D>::CH;
  if (HM && a.mask != nullptr && !kFwdThreeWaves<D, HP> && !streamed && a.B >= 2 && a.B <= kBalanceMaxB &&
      a.B * ((a.L + 31) / 32) <= 64 && a.ncu > 0 && grid == 2 * a.ncu && grid % 8 == 0) {
    const int per = grid / 8, unit = a.H * a.i_tiles;
    if (per % (2 * unit) == 0) a.balance = 1;
  }
  prof_begin(K_FWD, stream);
  bool resident = false;  // the pair bias held for the whole row (rows of one key tile)
  if constexpr (HP) resident = a.L <= KVTile<D>::CH;
  if constexpr (HP) {
    if (resident)
      hipLaunchKernelGGL((evo_fwd_kernel<T, D, HM, true, KVTile<D>::CH / 32>), dim3(grid), dim3(256), 0, stream, a);
  }
  if (!resident) hipLaunchKernelGGL((evo_fwd_kernel<T, D, HM, HP, 0>), dim3(grid), dim3(256), 0, stream, a);
  prof_end(K_FWD, stream);
  return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, hipStream_t s) {
  // rows of a length that is not a multiple of 32 take the mask path (with a
  // zero mask if none is given) so that keys past L are masked in the product
  const bool hm = a.mask != nullptr || (a.L % 32) != 0, hp = a.pair != nullptr;
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
