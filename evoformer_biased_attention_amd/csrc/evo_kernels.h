// Launch interfaces between the C-ABI layer and the kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace evo {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;  // [B,N,L] or null
  const uint16_t* pair;  // [B,H,L,L] or null
  uint16_t* out;
  float* lse;            // [B,N,H,L] or null (nothing kept for a backward)
  // element strides of dims B, N, L shared by q, k, v and out; the H heads of
  // D elements of one (b, n, l) row are dense
  int64_t sB, sN, sL;
  int B, N, L, H;
  int G;         // slices n per workgroup
  int n_groups;  // ceil(N / G)
  int i_tiles;   // query tiles per slice
  float scale;   // 1/sqrt(D)
  float sqrt_d;  // sqrt(D) in fp32 (the mask enters the score accumulator pre-multiplied by it)
  int ncu;       // compute units of the device
  int balance;   // 1: batch entries ordered by live length, long paired with short on each CU
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* mask;
  const uint16_t* pair;
  const uint16_t* out;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  uint16_t* dmask;       // [B,N,L] or null
  uint16_t* dpair;       // [B,H,L,L] or null
  float* delta;          // [B,N,H,L]
  float* dmask_part;     // [B,N,H,L]   (when dmask requested)
  float* dmask_f32;      // [B,N,L]
  float* dpair_part;     // [n_groups_q, B, H, L, L] (when dpair requested), one chunk's
  float* dpair_f32;      // [B,H,L,L]
  float* dq_part;        // [jtiles, B, q_nc, L,H,D] fp32 partials of dQ of one chunk of slices
                         // (rows longer than one key tile), dense
  // element strides of dims B, N, L shared by q, k, v, out, dout, dq, dk and
  // dv; the H heads of D elements of one (b, n, l) row are dense
  int64_t sB, sN, sL;
  int B, N, L, H;
  int Gq;          // slices per bwd_q3 workgroup
  int n_groups_q;  // bwd_q3 workgroups per (b, h, query tile) in the chunk
  // bwd_q3 covers the chunk of slices [q_n0, q_n0 + q_nc) (all N when rows
  // fit one key tile; longer rows go in chunks that bound the partials)
  int q_n0, q_nc;
  // the group slots of dpair_part hold running sums over the chunks: 0 for
  // the first chunk (bwd_q3 starts from zero), 1 after it (bwd_q3 starts from
  // the slot's sum the previous chunk left)
  int dpair_carry;
  int Gk;          // slices per bwd_kv3 workgroup
  int n_groups_k;
  float scale;
  float sqrt_d;    // sqrt(D) in fp32 (the masks enter the score accumulators pre-multiplied by it)
};

// Map a hardware workgroup id to a logical one so that consecutive logical
// ids run on the same XCD (the dispatcher deals ids round-robin over 8 XCDs).
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd;     // full rounds
  const int tail = total - per * kXcd;
  if (id >= per * kXcd) return id;  // ragged tail keeps its own order
  (void)tail;
  const int xcd = id % kXcd;
  const int slot = id / kXcd;
  return xcd * per + slot;
}

// Work order for batches whose entries differ in live length (padding masked
// with -inf).  A grid of exactly two workgroups per CU runs in one round, and
// xcd_remap gives XCD x the logical workgroups [x per, (x + 1) per), of which
// local slots j and j + per / 2 share a CU.  Work units (the `unit`
// consecutive workgroups of one (b, n-group)) are ranked from the costliest
// down; XCD x's first half of unit slots takes ranks x half .. x half + half - 1
// from the top, its second half the same count from the bottom, so each CU
// holds one costly and one cheap unit.  A bijection from logical unit slots to
// ranks when per is a multiple of 2 unit and the grid is 8 per.
__host__ __device__ inline int balanced_unit_rank(int lg, int per, int unit, int total_units) {
  const int x = lg / per, u = (lg % per) / unit;
  const int half = per / unit / 2;
  return u < half ? x * half + u : total_units - 1 - (x * half + (u - half));
}
constexpr int kBalanceMaxB = 8;  // batch entries ranked by one workgroup

hipError_t launch_fwd(FwdArgs a, int D, bool bf16, hipStream_t stream);
hipError_t launch_bwd(BwdArgs a, int D, bool bf16, hipStream_t stream);
// backward for rows that fit one key tile (L <= 256, or 128 at D = 64): bwd_q3 then bwd_kv3
hipError_t launch_bwd_tile(const BwdArgs& a, int D, bool bf16, hipStream_t stream);
// longer rows: part 0 is bwd_q3 over one chunk of slices with one key tile
// per workgroup (dQ left as fp32 partials), part 1 bwd_kv3 over query tiles,
// part 2 (no pair bias) bwd_q3 with all key tiles of a slice in one workgroup
hipError_t launch_bwd_q_split(const BwdArgs& a, int D, bool bf16, int part, hipStream_t stream);

}  // namespace evo
