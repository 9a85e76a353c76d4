// C ABI of the Evoformer attention library: argument checks, launch planning,
// workspace layout.  Declared in include/evo_attn.h.
//
// Interface rules follow the DeepSpeed4Science guide, §3.7: at most two
// biases, either may be absent; the bias shapes are [B,N,1,1,L] and
// [B,1,H,L,L]; inputs are fp16 or bf16 and must live on the current device;
// the backward supports head dims up to 64.  Where the guide's wrapper
// asserts, this layer returns a status code and enqueues nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/evo_attn.h"
#include "evo_kernels.h"
#include "evo_prof.h"

#include <algorithm>
#include <atomic>
#include <vector>

namespace {

constexpr int kMaxDevices = 64;

// -1 unknown, 0 not gfx950, 1 gfx950; and the device's compute units
int g_dev_ok[kMaxDevices];
int g_dev_cus[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

bool device_is_gfx950(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = 0;
    g_dev_cus[dev] = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) {
      g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
      g_dev_cus[dev] = prop.multiProcessorCount;
    }
  });
  return g_dev_ok[dev] == 1;
}

// compute units of a device that passed device_is_gfx950
int device_cus(int dev) { return (dev >= 0 && dev < kMaxDevices) ? g_dev_cus[dev] : 0; }

// ------------------------------------------------ static backward scratch
//
// The backward's workspace for evo_attn_bwd_noalloc (callers that cannot
// allocate device memory).  Every GPU the library runs on holds its own copy
// until the process ends; calls on one GPU share it, so calls that overlap on
// one GPU race.  Every byte a backward reads from it is written earlier in the
// same call, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = (size_t)EVO_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's copy of `scratch`, looked up once per device
// with that device current (the array's name is only a host-side stand-in).
void* g_scratch_ptr[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

void* scratch_device_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      p = nullptr;
    }
    g_scratch_ptr[dev] = p;
  });
  return g_scratch_ptr[dev];
}

struct Shape {
  int64_t B, N, L, H, D;
};

evo_status_t parse_shape(const int64_t* shape, int dtype, Shape* s) {
  if (shape == nullptr) return EVO_ERR_NULL_POINTER;
  if (dtype != EVO_F16 && dtype != EVO_BF16) return EVO_ERR_BAD_DTYPE;
  s->B = shape[0];
  s->N = shape[1];
  s->L = shape[2];
  s->H = shape[3];
  s->D = shape[4];
  if (s->B < 1 || s->N < 1 || s->L < 1 || s->H < 1 || s->D < 1) return EVO_ERR_BAD_SHAPE;
  if (s->D != 8 && s->D != 16 && s->D != 32 && s->D != 64) return EVO_ERR_HEAD_DIM;
  // every launch grid and per-slice index must fit 31 bits
  const int64_t lim = (int64_t)1 << 30;
  if (s->B > lim || s->N > lim || s->L > lim || s->H > lim) return EVO_ERR_BAD_SHAPE;
  if (s->L > 65536) return EVO_ERR_BAD_SHAPE;
  const double elems = (double)s->B * s->N * s->L * s->H * s->D;
  const double pair = (double)s->B * s->H * s->L * s->L;
  if (elems > 1e12 || pair > 1e12) return EVO_ERR_BAD_SHAPE;
  const double wgs = (double)s->B * s->N * s->H * ((s->L + 31) / 32);
  if (wgs > 2.0e9) return EVO_ERR_BAD_SHAPE;
  // the tile copies address a slice with 32-bit byte offsets
  if ((double)s->L * s->H * s->D * 2 >= 2147483648.0) return EVO_ERR_BAD_SHAPE;
  return EVO_OK;
}

// Element strides of dims B, N, L shared by the [B,N,L,H,D] tensors of a call
// (the H heads of D elements of one row are dense).  strides == nullptr: the
// dense layout.  Rows are 16-byte aligned (strides in multiples of 8
// elements), no two (b, n, l) rows overlap (over the dims of extent > 1 taken
// in increasing stride order, each stride covers the span of the ones below
// it, the first at least one row of H * D), and a (b, n) slice spans less
// than 2 GiB (the tile copies use 32-bit byte offsets).
struct Layout {
  int64_t sB, sN, sL;
};

evo_status_t parse_layout(const Shape& s, const int64_t* strides, Layout* lay) {
  const int64_t hd = s.H * s.D;
  if (strides == nullptr) {
    lay->sL = hd;
    lay->sN = s.L * hd;
    lay->sB = s.N * s.L * hd;
    return EVO_OK;
  }
  const int64_t st[3] = {strides[0], strides[1], strides[2]};
  const int64_t ext[3] = {s.B, s.N, s.L};
  for (int i = 0; i < 3; ++i)
    if (st[i] < 1 || st[i] > ((int64_t)1 << 40) || st[i] % 8 != 0) return EVO_ERR_BAD_STRIDES;
  int order[3] = {0, 1, 2};
  std::stable_sort(order, order + 3, [&](int x, int y) { return st[x] < st[y]; });
  double span = (double)hd;
  for (int k : order) {
    if (ext[k] == 1) continue;
    if ((double)st[k] < span) return EVO_ERR_BAD_STRIDES;
    span = (double)st[k] * (double)ext[k];
  }
  if ((double)(s.L - 1) * st[2] * 2 + (double)hd * 2 >= 2147483648.0) return EVO_ERR_BAD_STRIDES;
  const double foot = ((double)(s.B - 1) * st[0] + (double)(s.N - 1) * st[1] + (double)(s.L - 1) * st[2] + hd) * 2;
  if (foot > 1.0e15) return EVO_ERR_BAD_STRIDES;
  lay->sB = st[0];
  lay->sN = st[1];
  lay->sL = st[2];
  return EVO_OK;
}

// bytes from the first to one past the last element of a [B,N,L,H,D] tensor
int64_t footprint_bytes(const Shape& s, const Layout& l) {
  return ((s.B - 1) * l.sB + (s.N - 1) * l.sN + (s.L - 1) * l.sL + s.H * s.D) * 2;
}

evo_status_t check_device_ptr(const void* p, int dev) {
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return EVO_ERR_ALIGNMENT;
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next call
    return EVO_ERR_NOT_DEVICE_MEMORY;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return EVO_ERR_NOT_DEVICE_MEMORY;
  if (attr.device != dev) return EVO_ERR_NOT_DEVICE_MEMORY;
  return EVO_OK;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// any output overlapping any input or another output
bool any_alias(const Range* ins, int nin, const Range* outs, int nout) {
  for (int o = 0; o < nout; ++o) {
    if (outs[o].lo == 0) continue;
    for (int i = 0; i < nin; ++i)
      if (ins[i].lo != 0 && overlaps(outs[o], ins[i])) return true;
    for (int p = o + 1; p < nout; ++p)
      if (outs[p].lo != 0 && overlaps(outs[o], outs[p])) return true;
  }
  return false;
}

Range rng(const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo ? lo + (uintptr_t)bytes : 0};
}



// slices per forward workgroup: about two workgroups per CU (512), and never
// more than 4 slices each (measured on MI355X: larger groups lose more to the
// tail of the grid than they gain from reusing the pair bias)
int plan_fwd_group(const Shape& s) {
  const int64_t base = s.B * s.H * ((s.L + 127) / 128);
  int64_t g = (s.N * base) / 512;
  if (g < 1) g = 1;
  if (g > 4) g = 4;
  if (g > s.N) g = s.N;
  return (int)g;
}

// keys per backward tile (KVTile<D>::CH)
int64_t key_tile(int64_t D) { return D == 64 ? 128 : 256; }

// slices per bwd_q3 / bwd_kv3 workgroup (also the dpair partial count
// divisor).  A workgroup takes 128 rows and one key tile (all key tiles
// without a pair bias); one runs per CU (256 CUs).  The group count k is the
// smallest within 3% of the minimum of (rounds of workgroups) x (slices per
// workgroup): fewer groups mean fewer dpair partials and fewer per-workgroup
// set-ups.
int plan_bwdq_group(const Shape& s, bool has_pair) {
  const int64_t jtiles = (s.L + key_tile(s.D) - 1) / key_tile(s.D);
  // without a pair bias a workgroup walks every key tile of its slices
  const int64_t per_group = s.B * s.H * ((s.L + 127) / 128) * (has_pair ? jtiles : 1);
  const int64_t kmax = s.N < 4096 ? s.N : 4096;
  auto cost = [&](int64_t k) { return ((per_group * k + 255) / 256) * ((s.N + k - 1) / k); };
  int64_t best_t = INT64_MAX;
  for (int64_t k = 1; k <= kmax; ++k) best_t = std::min(best_t, cost(k));
  int64_t k = 1;
  while (k < kmax && cost(k) * 100 > best_t * 103) ++k;
  int64_t g = (s.N + k - 1) / k;
  // rows longer than one key tile without a pair bias (no dpair partials to
  // multiply; a workgroup walks all key tiles of its slices): at most 24 key
  // tiles per workgroup, so the grid runs in more, shorter rounds (measured on
  // MI355X at (1,384,512,8,32): bwd_q3 293 us at 24, 296 at 48, 304 at 96)
  constexpr int64_t kMaxTilesPerGroup = 24;
  if (jtiles > 1 && !has_pair && g * jtiles > kMaxTilesPerGroup) g = std::max<int64_t>(1, kMaxTilesPerGroup / jtiles);
  return (int)g;
}

// slices per bwd_kv3 workgroup: same rule over the key-side grid (one
// workgroup per 128 keys and slice group)
int plan_bwdkv_group(const Shape& s) {
  const int64_t per_group = s.B * s.H * ((s.L + 127) / 128);
  const int64_t kmax = s.N < 4096 ? s.N : 4096;
  auto cost = [&](int64_t k) { return ((per_group * k + 255) / 256) * ((s.N + k - 1) / k); };
  int64_t best_t = INT64_MAX;
  for (int64_t k = 1; k <= kmax; ++k) best_t = std::min(best_t, cost(k));
  int64_t k = 1;
  while (k < kmax && cost(k) * 100 > best_t * 103) ++k;
  int64_t g = (s.N + k - 1) / k;
  // rows longer than one key tile (the query tiles walked per slice): groups
  // of at most 8 slices (measured on MI355X: 383 -> 357 us at (1,384,512,8,32),
  // 1287 -> 1174 us at (1,768,768,4,32); rows of one tile keep the rule above)
  if (s.L > key_tile(s.D) && g > 8) g = 8;
  return (int)g;
}

// bwd_q3 plan: slices per workgroup (gq), workgroups per (b, h, query tile,
// key tile) in a chunk (ngq, also the dpair group slots) and slices per chunk
// (nc).  Rows of one key tile take all slices at once (no dQ partials).
// Longer rows keep their fp32 partials (dQ per key tile of the chunk's slices,
// plus the dpair slots) within a byte budget: the one-chunk plan when it fits,
// else, of the chunkings and group counts that fit, the first in a fixed order
// (modelled time: chunks x workgroup rounds x (slices per workgroup + 4, the
// set-up of a workgroup in slice units); then fewer chunks, then fewer
// groups), else one slice at a time (the least workspace the backward can run
// in).  The order does not depend on the budget, so a plan chosen for one
// budget is chosen again for any smaller budget it still fits.
struct BwdQPlan {
  int gq, ngq, nc;
};
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdQPlan plan_bwdq(const Shape& s, bool has_pair, size_t budget) {
  const int64_t jtiles = (s.L + key_tile(s.D) - 1) / key_tile(s.D);
  const int64_t g1 = plan_bwdq_group(s, has_pair);
  const int64_t k1 = (s.N + g1 - 1) / g1;
  // rows of one key tile, and longer rows without a pair bias (a workgroup
  // walks all key tiles and keeps dQ in registers): no partials, one chunk
  if (jtiles == 1 || !has_pair) return {(int)g1, (int)k1, (int)s.N};
  const size_t dq_slice = (size_t)jtiles * s.B * s.L * s.H * s.D * sizeof(float);
  const size_t slot = has_pair ? (size_t)s.B * s.H * s.L * s.L * sizeof(float) : 0;
  auto bytes = [&](int64_t nc, int64_t k) { return al256((size_t)nc * dq_slice) + al256((size_t)k * slot); };
  if (bytes(s.N, k1) <= budget) return {(int)g1, (int)k1, (int)s.N};
  const int64_t per_group = s.B * s.H * ((s.L + 127) / 128) * jtiles;
  struct Cand {
    int64_t cost, chunks, k, g, nc;
  };
  std::vector<Cand> cands;
  const int64_t cmax = std::min<int64_t>(s.N, 64);
  for (int64_t c = 1; c <= cmax; ++c) {
    const int64_t nc = (s.N + c - 1) / c;
    if ((s.N + nc - 1) / nc != c) continue;  // the same chunking as a smaller count
    for (int64_t k = 1; k <= std::min<int64_t>(nc, 64); ++k) {
      const int64_t g = (nc + k - 1) / k;
      if ((nc + g - 1) / g != k) continue;  // k groups of g slices do not form
      if (!has_pair && g > 24) continue;    // as plan_bwdq_group
      if (bytes(nc, k) > budget) continue;
      cands.push_back({c * ((per_group * k + 255) / 256) * (g + 4), c, k, g, nc});
    }
  }
  if (cands.empty()) return {1, 1, 1};
  const Cand* pick = &cands[0];
  for (const Cand& x : cands) {
    if (x.cost != pick->cost ? x.cost < pick->cost
                             : (x.chunks != pick->chunks ? x.chunks < pick->chunks : x.k < pick->k))
      pick = &x;
  }
  return {(int)pick->g, (int)pick->k, (int)pick->nc};
}

// Partial budget of a workspace sized by evo_attn_bwd_workspace_bytes (A/B on
// one MI355X, (1,768,768,4,32) bf16 step: unchunked 3.96 ms; 640 MiB +1.8%,
// 384 MiB +3.9%, 160 MiB +12%; (1,384,512,8,32) unchanged from 384 MiB up)
constexpr size_t kDefaultPartialBudget = (size_t)384 << 20;

// Workspace: the regions whose size does not depend on the plan first (so
// their offsets do not either), then the dpair group slots and dQ partials.
struct WsLayout {
  size_t delta, dmask_part, dmask_f32, dpair_f32, fixed, dpair_part, dq_part, total;
  int gq, ngq, nc;
};

WsLayout ws_layout(const Shape& s, bool has_mask, bool has_pair, size_t budget) {
  WsLayout w;
  const size_t rows = (size_t)s.B * s.N * s.H * s.L * sizeof(float);
  const size_t per = (size_t)s.B * s.H * s.L * s.L * sizeof(float);
  size_t off = 0;
  w.delta = off;
  off += al256(rows);
  w.dmask_part = w.dmask_f32 = (size_t)-1;
  if (has_mask) {
    w.dmask_part = off;
    off += al256(rows);
    w.dmask_f32 = off;
    off += al256((size_t)s.B * s.N * s.L * sizeof(float));
  }
  w.dpair_f32 = (size_t)-1;
  if (has_pair) {
    w.dpair_f32 = off;
    off += al256(per);
  }
  w.fixed = off;
  const BwdQPlan qp = plan_bwdq(s, has_pair, budget);
  w.gq = qp.gq;
  w.ngq = qp.ngq;
  w.nc = qp.nc;
  w.dpair_part = (size_t)-1;
  if (has_pair) {
    w.dpair_part = off;
    off += al256(per * (size_t)w.ngq);
  }
  // fp32 partials of dQ of one chunk of slices, one per key tile, when a row
  // spans several tiles and the query side splits it by key tile (with a pair bias)
  w.dq_part = (size_t)-1;
  const int64_t jtiles = (s.L + key_tile(s.D) - 1) / key_tile(s.D);
  if (jtiles > 1 && has_pair) {
    w.dq_part = off;
    off += al256((size_t)jtiles * s.B * w.nc * s.L * s.H * s.D * sizeof(float));
  }
  w.total = off;
  return w;
}

// The layout for a workspace of `bytes`: the plan that fits what is left
// after the fixed regions.
WsLayout ws_layout_within(const Shape& s, bool has_mask, bool has_pair, size_t bytes) {
  const size_t fixed = ws_layout(s, has_mask, has_pair, 0).fixed;
  return ws_layout(s, has_mask, has_pair, bytes > fixed ? bytes - fixed : 0);
}

}  // namespace


// ------------------------------------------------------------ instrumentation

namespace evo {
namespace {
std::atomic<int> g_prof_on{0};
std::mutex g_prof_mu;
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::vector<hipEvent_t> g_prof_pool;  // free events
std::vector<ProfRec> g_prof_recs;     // recorded launches not yet read
constexpr size_t kProfMaxRecs = 1 << 16;
int g_prof_open_kind = -1;
hipEvent_t g_prof_open_ev = nullptr;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void prof_begin(KernelKind k, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_recs.size() >= kProfMaxRecs) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {  // no record for this launch
    (void)hipGetLastError();
    g_prof_pool.push_back(e);
    return;
  }
  g_prof_open_kind = (int)k;
  g_prof_open_ev = e;
}

void prof_end(KernelKind k, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_open_kind != (int)k || !g_prof_open_ev) return;
  hipEvent_t e = prof_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {  // drop the open record
    (void)hipGetLastError();
    g_prof_pool.push_back(e);
    g_prof_pool.push_back(g_prof_open_ev);
  } else {
    g_prof_recs.push_back(ProfRec{(int)k, g_prof_open_ev, e});
  }
  g_prof_open_kind = -1;
  g_prof_open_ev = nullptr;
}
}  // namespace evo

extern "C" {

const char* evo_status_string(int status) {
  switch (status) {
    case EVO_OK: return "ok";
    case EVO_ERR_NULL_POINTER: return "a required pointer is NULL (or a bias gradient was requested without its bias)";
    case EVO_ERR_BAD_SHAPE: return "bad shape: every dimension must be >= 1 and within the supported size";
    case EVO_ERR_BAD_DTYPE: return "bad dtype: expected EVO_F16 or EVO_BF16";
    case EVO_ERR_HEAD_DIM: return "head dim D must be 8, 16, 32 or 64";
    case EVO_ERR_ALIGNMENT: return "a tensor pointer is not 16-byte aligned";
    case EVO_ERR_NOT_DEVICE_MEMORY: return "a tensor pointer is not device memory of the current device";
    case EVO_ERR_WORKSPACE: return "workspace missing or too small";
    case EVO_ERR_DEVICE: return "the current device is not gfx950 (MI355X)";
    case EVO_ERR_LAUNCH: return "kernel launch failed";
    case EVO_ERR_ALIAS: return "an output overlaps an input or another output";
    case EVO_ERR_BAD_STRIDES: return "strides: not multiples of 8 elements, overlapping rows, or a slice past 2 GiB";
    case EVO_ERR_SCRATCH_LIMIT:
      return "evo_attn_bwd_noalloc: this backward needs more scratch than the library's static limit "
             "(EVO_NOALLOC_SCRATCH_BYTES); call evo_attn_bwd with a workspace instead";
  }
  return "unknown status";
}

evo_status_t evo_attn_fwd(const void* q, const void* k, const void* v, const void* mask_bias, const void* pair_bias,
                          void* out, float* lse, const int64_t shape[5], int dtype, void* stream) {
  return evo_attn_fwd_strided(q, k, v, mask_bias, pair_bias, out, lse, shape, nullptr, dtype, stream);
}

evo_status_t evo_attn_fwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, void* out, float* lse, const int64_t shape[5],
                                  const int64_t strides[3], int dtype, void* stream) {
  Shape s;
  evo_status_t st = parse_shape(shape, dtype, &s);
  if (st != EVO_OK) return st;
  Layout lay;
  if ((st = parse_layout(s, strides, &lay)) != EVO_OK) return st;
  // lse may be NULL: a forward with no backward after it (inference)
  if (!q || !k || !v || !out) return EVO_ERR_NULL_POINTER;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EVO_ERR_DEVICE;
  if (!device_is_gfx950(dev)) return EVO_ERR_DEVICE;
  const void* ptrs[] = {q, k, v, mask_bias, pair_bias, out, lse};
  for (const void* p : ptrs)
    if (p && (st = check_device_ptr(p, dev)) != EVO_OK) return st;
  const int64_t tb = footprint_bytes(s, lay);
  const Range ins[] = {rng(q, tb), rng(k, tb), rng(v, tb), rng(mask_bias, s.B * s.N * s.L * 2),
                       rng(pair_bias, s.B * s.H * s.L * s.L * 2)};
  const Range outs[] = {rng(out, tb), rng(lse, s.B * s.N * s.H * s.L * 4)};
  if (any_alias(ins, 5, outs, 2)) return EVO_ERR_ALIAS;

  evo::FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.mask = static_cast<const uint16_t*>(mask_bias);
  a.pair = static_cast<const uint16_t*>(pair_bias);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.sB = lay.sB;
  a.sN = lay.sN;
  a.sL = lay.sL;
  a.B = (int)s.B;
  a.N = (int)s.N;
  a.L = (int)s.L;
  a.H = (int)s.H;
  a.G = plan_fwd_group(s);
  a.scale = (float)(1.0 / std::sqrt((double)s.D));
  a.sqrt_d = (float)std::sqrt((double)s.D);
  a.ncu = device_cus(dev);
  hipError_t e = evo::launch_fwd(a, (int)s.D, dtype == EVO_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EVO_OK : EVO_ERR_LAUNCH;
}

size_t evo_attn_bwd_workspace_bytes(const int64_t shape[5], int dtype, int has_mask, int has_pair) {
  Shape s;
  if (parse_shape(shape, dtype, &s) != EVO_OK) return 0;
  return ws_layout(s, has_mask != 0, has_pair != 0, kDefaultPartialBudget).total;
}

size_t evo_attn_bwd_workspace_bytes_within(const int64_t shape[5], int dtype, int has_mask, int has_pair,
                                           size_t partial_budget) {
  Shape s;
  if (parse_shape(shape, dtype, &s) != EVO_OK) return 0;
  return ws_layout(s, has_mask != 0, has_pair != 0, partial_budget).total;
}

evo_status_t evo_attn_bwd_workspace_offsets(const int64_t shape[5], int dtype, int has_mask, int has_pair,
                                            size_t* off_delta, size_t* off_dmask_f32, size_t* off_dpair_f32) {
  Shape s;
  evo_status_t st = parse_shape(shape, dtype, &s);
  if (st != EVO_OK) return st;
  WsLayout w = ws_layout(s, has_mask != 0, has_pair != 0, 0);  // offsets do not depend on the plan
  if (off_delta) *off_delta = w.delta;
  if (off_dmask_f32) *off_dmask_f32 = w.dmask_f32;
  if (off_dpair_f32) *off_dpair_f32 = w.dpair_f32;
  return EVO_OK;
}

evo_status_t evo_attn_bwd(const void* q, const void* k, const void* v, const void* mask_bias, const void* pair_bias,
                          const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                          void* dmask_bias, void* dpair_bias, void* workspace, size_t workspace_bytes,
                          const int64_t shape[5], int dtype, void* stream) {
  return evo_attn_bwd_strided(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias,
                              workspace, workspace_bytes, shape, nullptr, dtype, stream);
}

}  // extern "C"

namespace {

// The backward behind evo_attn_bwd_strided and evo_attn_bwd_noalloc.  With
// use_scratch the workspace is this GPU's copy of the static `scratch` array
// (workspace and workspace_bytes are ignored).
evo_status_t bwd_impl(const void* q, const void* k, const void* v, const void* mask_bias, const void* pair_bias,
                      const void* out, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* dmask_bias, void* dpair_bias, void* workspace, size_t workspace_bytes,
                      const int64_t shape[5], const int64_t strides[3], int dtype, void* stream, bool use_scratch) {
  Shape s;
  evo_status_t st = parse_shape(shape, dtype, &s);
  if (st != EVO_OK) return st;
  Layout lay;
  if ((st = parse_layout(s, strides, &lay)) != EVO_OK) return st;
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return EVO_ERR_NULL_POINTER;
  if ((dmask_bias && !mask_bias) || (dpair_bias && !pair_bias)) return EVO_ERR_NULL_POINTER;
  const bool has_mask = mask_bias != nullptr, has_pair = pair_bias != nullptr;
  // the plan that fits the workspace given (the static scratch for noalloc)
  const WsLayout w = ws_layout_within(s, has_mask, has_pair, use_scratch ? kScratchBytes : workspace_bytes);
  if (use_scratch) {
    if (w.total > kScratchBytes) return EVO_ERR_SCRATCH_LIMIT;
  } else if (!workspace || workspace_bytes < w.total) {
    return EVO_ERR_WORKSPACE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EVO_ERR_DEVICE;
  if (!device_is_gfx950(dev)) return EVO_ERR_DEVICE;
  const void* ptrs[] = {q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias};
  for (const void* p : ptrs)
    if (p && (st = check_device_ptr(p, dev)) != EVO_OK) return st;
  if (use_scratch) {
    workspace = scratch_device_ptr(dev);
    if (workspace == nullptr) return EVO_ERR_DEVICE;
    workspace_bytes = kScratchBytes;
  } else if ((st = check_device_ptr(workspace, dev)) != EVO_OK) {
    return st;
  }
  const int64_t tb = footprint_bytes(s, lay);
  const Range ins[] = {rng(q, tb),
                       rng(k, tb),
                       rng(v, tb),
                       rng(mask_bias, s.B * s.N * s.L * 2),
                       rng(pair_bias, s.B * s.H * s.L * s.L * 2),
                       rng(out, tb),
                       rng(lse, s.B * s.N * s.H * s.L * 4),
                       rng(dout, tb)};
  const Range outs[] = {rng(dq, tb),
                        rng(dk, tb),
                        rng(dv, tb),
                        rng(dmask_bias, s.B * s.N * s.L * 2),
                        rng(dpair_bias, s.B * s.H * s.L * s.L * 2),
                        rng(workspace, (int64_t)w.total)};
  if (any_alias(ins, 8, outs, 6)) return EVO_ERR_ALIAS;

  char* ws = static_cast<char*>(workspace);
  evo::BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.mask = static_cast<const uint16_t*>(mask_bias);
  a.pair = static_cast<const uint16_t*>(pair_bias);
  a.out = static_cast<const uint16_t*>(out);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.dmask = static_cast<uint16_t*>(dmask_bias);
  a.dpair = static_cast<uint16_t*>(dpair_bias);
  a.delta = reinterpret_cast<float*>(ws + w.delta);
  a.dmask_part = has_mask ? reinterpret_cast<float*>(ws + w.dmask_part) : nullptr;
  a.dmask_f32 = has_mask ? reinterpret_cast<float*>(ws + w.dmask_f32) : nullptr;
  a.dpair_part = has_pair ? reinterpret_cast<float*>(ws + w.dpair_part) : nullptr;
  a.dpair_f32 = has_pair ? reinterpret_cast<float*>(ws + w.dpair_f32) : nullptr;
  a.dq_part = (w.dq_part != (size_t)-1) ? reinterpret_cast<float*>(ws + w.dq_part) : nullptr;
  a.sB = lay.sB;
  a.sN = lay.sN;
  a.sL = lay.sL;
  a.B = (int)s.B;
  a.N = (int)s.N;
  a.L = (int)s.L;
  a.H = (int)s.H;
  a.Gq = w.gq;
  a.n_groups_q = w.ngq;
  a.q_n0 = 0;
  a.q_nc = w.nc;
  a.dpair_carry = 0;
  a.Gk = plan_bwdkv_group(s);
  a.n_groups_k = (int)((s.N + a.Gk - 1) / a.Gk);
  a.sqrt_d = (float)std::sqrt((double)s.D);
  a.scale = (float)(1.0 / std::sqrt((double)s.D));
  hipError_t e = evo::launch_bwd(a, (int)s.D, dtype == EVO_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? EVO_OK : EVO_ERR_LAUNCH;
}

}  // namespace

extern "C" {

evo_status_t evo_attn_bwd_strided(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias, void* workspace,
                                  size_t workspace_bytes, const int64_t shape[5], const int64_t strides[3],
                                  int dtype, void* stream) {
  return bwd_impl(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, workspace,
                  workspace_bytes, shape, strides, dtype, stream, false);
}

evo_status_t evo_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* mask_bias,
                                  const void* pair_bias, const void* out, const float* lse, const void* dout,
                                  void* dq, void* dk, void* dv, void* dmask_bias, void* dpair_bias,
                                  const int64_t shape[5], const int64_t strides[3], int dtype, void* stream) {
  return bwd_impl(q, k, v, mask_bias, pair_bias, out, lse, dout, dq, dk, dv, dmask_bias, dpair_bias, nullptr, 0,
                  shape, strides, dtype, stream, true);
}

int evo_attn_profile_enable(int on) {
  int prev = evo::g_prof_on.exchange(on ? 1 : 0);
  return prev;
}

evo_status_t evo_attn_profile_read(double total_ms[EVO_PROFILE_KINDS], int64_t launches[EVO_PROFILE_KINDS]) {
  if (!total_ms || !launches) return EVO_ERR_NULL_POINTER;
  std::lock_guard<std::mutex> lk(evo::g_prof_mu);
  for (int k = 0; k < EVO_PROFILE_KINDS; ++k) {
    total_ms[k] = 0.0;
    launches[k] = 0;
  }
  evo_status_t st = EVO_OK;
  for (auto& r : evo::g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      (void)hipGetLastError();
      st = EVO_ERR_LAUNCH;
    } else if (r.kind >= 0 && r.kind < EVO_PROFILE_KINDS) {
      total_ms[r.kind] += ms;
      launches[r.kind] += 1;
    }
    evo::g_prof_pool.push_back(r.a);
    evo::g_prof_pool.push_back(r.b);
  }
  evo::g_prof_recs.clear();
  return st;
}

const char* evo_attn_profile_kernel_name(int kind) {
  switch (kind) {
    case evo::K_FWD: return "fwd";
    case evo::K_BWD_PRE: return "bwd_pre";
    case evo::K_BWD_KV: return "bwd_kv";
    case evo::K_BWD_Q: return "bwd_q";
    case evo::K_BWD_FIN: return "bwd_fin";
  }
  return "unknown";
}

}  // extern "C"
