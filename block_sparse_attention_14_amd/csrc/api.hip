// C ABI entry points: argument validation (entirely on the host, before any
// launch), then kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "kernels.h"
#include "sol_attn.h"

namespace {

// Device memory of sol_attn_forward_noalloc: the pooled keys and values and
// the forward's workspace of one call, for callers that cannot allocate. One
// copy per GPU, at its own address, held until the process ends. In host
// code `scratch` names a host-side stand-in: its device address on the
// current GPU comes from hipGetSymbolAddress (scratch_base below), and only
// that address is ever handed to a kernel or a runtime call.
__device__ __align__(256) unsigned char scratch[SOL_ATTN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices] = {nullptr};

// The device address of `scratch` on the current GPU, looked up once per
// device with that device current; SOL_EHIP if the runtime refuses.
int scratch_base(void** base) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SOL_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return SOL_EHIP;
    scratch_dev[dev] = p;
  }
  *base = scratch_dev[dev];
  return SOL_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: [header words | the plan's item and unit counts | item costs |
// item order | work units | pooled-key copies and statistics of the optional
// modes]. The cost and order slots are sized for items of two query blocks,
// the most items any group size gives; the units for every pair of every
// item of any group size (at most ceil(Nq / 2) + 8 per head).
struct WsLayout {
  size_t plan, cost, perm, units, qpool, kh, km, kl, vt, vbar16, kstats, kmom, total;
};

// Key blocks per head in the tiled operand planes: Nk rounded up to 64 (the
// pre-pass writes the padding as zeros, so no read of a plane needs a bound).
int padded_blocks(int Nk) { return (Nk + 63) / 64 * 64; }

WsLayout ws_layout(int BH, int N, int d) {
  const size_t Nq = (size_t)(N + 63) / 64;
  const size_t items = (size_t)sol::forward_items(BH, (int)Nq, 2);
  const size_t plane = round_up((size_t)BH * Nq * (size_t)d * 2, 256);
  const size_t tplane = round_up((size_t)BH * (size_t)d * (size_t)padded_blocks((int)Nq) * 2, 256);
  WsLayout w;
  w.plan = round_up(sol::kHdrWords * 4, 256);
  w.cost = w.plan + 256;
  w.perm = round_up(w.cost + 4 * items, 256);
  w.units = round_up(w.perm + 4 * items, 256);
  w.qpool = round_up(w.units + 4 * (size_t)BH * ((Nq + 1) / 2 + 8), 256);
  w.kh = round_up(w.qpool + (size_t)BH * Nq * (size_t)d * 4, 256);
  w.km = w.kh + tplane;
  w.kl = w.km + tplane;
  w.vt = w.kl + tplane;
  w.vbar16 = w.vt + tplane;
  w.kstats = w.vbar16 + plane;
  w.kmom = round_up(w.kstats + (size_t)BH * 2 * (size_t)d * 4, 256);
  w.total = round_up(w.kmom + (size_t)BH * (size_t)(d + 1) * (size_t)d * 4, 256);
  return w;
}

// Query blocks per work item of the fused kernel. Larger groups read the
// head's pooled keys and values once for more query blocks (the routing
// pass's traffic falls as 1/G, and with 16 blocks every column of its score
// tiles is a block), smaller ones give the persistent grid more items to
// balance; a group is taken only while the call keeps at least 6 items per
// CU (three per workgroup), and eight or sixteen blocks only up to 2048 key
// blocks (their kept bits must fit the workgroup's LDS). Where the routing
// pass dominates the items (row-max routing with tau <= 4) the largest of
// 16, 8 and 6 that still gives 4 items per CU is taken: on the 119K-token
// video layer sixteen are 12% faster than eight at tau = 2 and 3% at tau = 4,
// but 9% slower at tau = 8, where larger items balance worse; on the
// 32K-token layer six are 5% faster than four at tau = 2 to 4 (and 5%
// slower on its variant with six diffuse heads, whose kept work dominates).
// A flag may ask for a size; none there means this automatic choice.
std::mutex cu_mu;
int cu_count[64] = {0};

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(cu_mu);
  if (cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    cu_count[dev] = n;
  }
  return cu_count[dev];
}

constexpr float kGroup16MaxTau = 4.f;

// A planned item whose estimated cost (the sizes of its pairs' unions, in
// key blocks) reaches a quarter of the head's key blocks is handed out pair
// by pair: its routing pass, a stream over all Nk pooled blocks, is then a
// small part of each pair (at tau = 8 on the 32K-token layer typical items
// cost about Nk / 8; items of heads that keep every block, 2 Nk).
unsigned split_cost(int Nk) { return (unsigned)std::max(1, Nk / 4); }

int auto_group(int BH, int Nq, const sol_attn_route& r) {
  const long long target = 6ll * device_cus();
  if (r.rule == SOL_ROUTE_ROWMAX && r.tau <= kGroup16MaxTau) {
    // routing dominates: larger groups while there are 4 items per CU
    const long long low = 4ll * device_cus();
    if (Nq <= sol::kMaxKeyBlocksG8 && (long long)sol::forward_items(BH, Nq, 16) >= low) return 16;
    if (Nq <= sol::kMaxKeyBlocksG8 && (long long)sol::forward_items(BH, Nq, 8) >= low) return 8;
    if ((long long)sol::forward_items(BH, Nq, 6) >= low) return 6;
  }
  if (Nq <= sol::kMaxKeyBlocksG8 && (long long)sol::forward_items(BH, Nq, 8) >= target) return 8;
  if ((long long)sol::forward_items(BH, Nq, 4) >= target) return 4;
  return 2;
}

// The group size a flag field asks for (0: automatic), or 0 if unsupported.
int group_of(unsigned flags, int BH, int Nq, const sol_attn_route& r) {
  if (flags & SOL_F_GROUP16) return Nq <= sol::kMaxKeyBlocksG8 ? 16 : 0;
  if (flags & SOL_F_GROUP6) return 6;
  switch ((flags & SOL_F_GROUP_MASK) >> SOL_F_GROUP_SHIFT) {
    case 1: return 2;
    case 2: return 4;
    case 3: return Nq <= sol::kMaxKeyBlocksG8 ? 8 : 0;
    default: return auto_group(BH, Nq, r);
  }
}

// Items beyond this are taken in sequence order (the one-workgroup sort
// would cost more than the balance it buys).
constexpr int kMaxOrderedItems = 1 << 20;

bool use_order(float tau, int nitems) { return !isinf(tau) && nitems > 1 && nitems <= kMaxOrderedItems; }

// The forward plans its work order by itself only where the order was
// measured to repay the planning kernels (about 25 us on the 32K-token video
// layer, growing with B*H*Nq*Nk): row-max routing with tau >= 8, where the
// budgets of the query blocks spread widest; at most about eight items per
// workgroup of the persistent grid, where one heavy item started late sets
// the finish (with more, the dynamic queues balance the work by themselves);
// and at least 2^21 query-block x key-block pairs, so that the extra launches
// are small against the call. Measured whole calls, planned vs in sequence:
// 32K layer tau = 8 -8%, tau = 16 -5%, tau = 6 +1%; 119K layer tau = 8 +9%;
// 4K image layer tau = 8 +12%.
constexpr float kPlanMinTau = 8.f;
constexpr int kPlanMaxItems = 4096;
constexpr long long kPlanMinPairs = 1ll << 21;

// Largest B * H of the launches whose grid has one row per head (plan, masks).
constexpr int kMaxGridHeads = 65535;

bool plan_by_default(const sol_attn_route& r, int BH, int Nq, int nitems, int group) {
  return group == auto_group(BH, Nq, r) && r.rule == SOL_ROUTE_ROWMAX && r.tau >= kPlanMinTau &&
         use_order(r.tau, nitems) && nitems <= kPlanMaxItems && (long long)BH * Nq * Nq >= kPlanMinPairs &&
         BH <= kMaxGridHeads;
}

int check_sizes(int B, int H, int N, int d, int Bq, int Bk) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return SOL_EINVAL;
  if (d != 64 && d != 128) return SOL_EUNSUPPORTED;
  if (Bq != 64 || Bk != 64) return SOL_EUNSUPPORTED;
  if (N > SOL_ATTN_MAX_N) return SOL_EUNSUPPORTED;
  const long long nq = (N + 63) / 64;
  if ((long long)B * H * nq > (1ll << 30)) return SOL_EUNSUPPORTED;  // ticket space
  return SOL_OK;
}

int check_tau(float tau) { return (isnan(tau) || tau < 0.f) ? SOL_EINVAL : SOL_OK; }

sol_attn_route rowmax_route(float tau) {
  sol_attn_route r;
  r.rule = SOL_ROUTE_ROWMAX;
  r.tau = tau;
  r.beta = 0.f;
  r.sink_first = 0;
  r.sink_count = 0;
  return r;
}

// Planning: per-item costs and the order of each queue into the workspace
// (row-max rule, finite tau, sizes the sort handles), else the identity
// order, which every later planned forward may still read. The items are
// those of the automatic group size.
hipError_t plan_impl(const uint16_t* q, const float* kpool, int BH, int N, int d, float tau, void* ws, hipStream_t s,
                     bool* ordered) {
  const WsLayout w = ws_layout(BH, N, d);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  const int Nq = (N + 63) / 64, Nk = Nq;
  unsigned* perm = reinterpret_cast<unsigned*>(wsb + w.perm);
  unsigned* units = reinterpret_cast<unsigned*>(wsb + w.units);
  unsigned* plan_items = reinterpret_cast<unsigned*>(wsb + w.plan);
  const int group = auto_group(BH, Nq, rowmax_route(tau));
  const int nitems = sol::forward_items(BH, Nq, group);
  *ordered = use_order(tau, nitems) && BH <= kMaxGridHeads;
  if (*ordered)
    return sol::launch_plan(q, kpool, reinterpret_cast<unsigned*>(wsb + w.cost), perm, units, plan_items, BH, N, Nq,
                            Nk, d, tau, (float)(1.0 / sqrt((double)d)), group, split_cost(Nk), s);
  return sol::launch_identity_order(units, plan_items, nitems, group, s);
}

int check_route(const sol_attn_route& r, int N, int Bk) {
  if (r.rule == SOL_ROUTE_ROWMAX) {
    if (check_tau(r.tau) != SOL_OK) return SOL_EINVAL;
  } else if (r.rule == SOL_ROUTE_GAUSS || r.rule == SOL_ROUTE_GAUSS_DIAG) {
    if (!isfinite(r.beta)) return SOL_EINVAL;
  } else {
    return SOL_EINVAL;
  }
  if (r.sink_count < 0) return SOL_EINVAL;
  if (r.sink_count > 0) {
    const long long nk = Bk > 0 ? (N + (long long)Bk - 1) / Bk : 0;
    if (r.sink_first < 0 || (long long)r.sink_first + r.sink_count > nk) return SOL_EINVAL;
  }
  return SOL_OK;
}

// Everything of a forward but the caller's pooled buffers and workspace.
int check_args(const void* q, const void* k, const void* v, const void* out, int B, int H, int N, int d, int Bq,
               int Bk, const sol_attn_route& route, unsigned flags, const sol_attn_stats* stats) {
  if (!q || !k || !v || !out) return SOL_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(stats, 8))
    return SOL_EINVAL;
  if (check_route(route, N, Bk) != SOL_OK) return SOL_EINVAL;
  if (flags & ~(unsigned)(SOL_F_POOLED | SOL_F_EXACT_ONLY | SOL_F_PLANNED | SOL_F_ROW_CORRECTION | SOL_F_OUT_BF16 |
                          SOL_F_GROUP_MASK | SOL_F_GROUP16 | SOL_F_GROUP6 | SOL_F_PREPARED))
    return SOL_EINVAL;
  // one group size at most; a plan orders the items of the automatic size
  const int nsizes = ((flags & SOL_F_GROUP_MASK) != 0) + ((flags & SOL_F_GROUP16) != 0) + ((flags & SOL_F_GROUP6) != 0);
  if (nsizes > 1) return SOL_EINVAL;
  if ((flags & SOL_F_PLANNED) && nsizes > 0) return SOL_EINVAL;
  if ((flags & SOL_F_EXACT_ONLY) && (flags & SOL_F_ROW_CORRECTION)) return SOL_EINVAL;
  // exact-only under a Gaussian threshold: a query block whose threshold lies
  // above its best block would keep nothing, and its rows would have no terms
  if ((flags & SOL_F_EXACT_ONLY) && route.rule != SOL_ROUTE_ROWMAX && route.sink_count == 0) return SOL_EINVAL;
  if ((flags & (SOL_F_PLANNED | SOL_F_PREPARED)) && !(flags & SOL_F_POOLED)) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, Bq, Bk);
  if (rc != SOL_OK) return rc;
  // eight or sixteen query blocks per item only up to kMaxKeyBlocksG8 key blocks
  if ((((flags & SOL_F_GROUP_MASK) >> SOL_F_GROUP_SHIFT) == 3 || (flags & SOL_F_GROUP16)) &&
      (N + 63) / 64 > sol::kMaxKeyBlocksG8)
    return SOL_EUNSUPPORTED;
  return SOL_OK;
}

int check_forward(const void* q, const void* k, const void* v, const void* out, int B, int H, int N,
                  int d, int Bq, int Bk, const sol_attn_route& route, unsigned flags, const sol_attn_stats* stats,
                  const float* kpool, const float* vmean, const void* ws, size_t ws_bytes) {
  if (!kpool || !vmean || !ws) return SOL_EINVAL;
  if (!aligned(kpool, 16) || !aligned(vmean, 16) || !aligned(ws, 256)) return SOL_EINVAL;
  const int rc = check_args(q, k, v, out, B, H, N, d, Bq, Bk, route, flags, stats);
  if (rc != SOL_OK) return rc;
  if (ws_bytes < sol_attn_workspace_bytes(B, H, N, d, Bq, Bk)) return SOL_EWORKSPACE;
  return SOL_OK;
}

// The pooling pre-pass of a forward: the pooled queries always (the routing
// pass reads them), the pooled keys and values when k16 and v16 are given
// (else the caller's kpool and vmean are read), and from those means the
// routing pass's bf16 operand planes (and, for the per-row correction, its
// row-major bf16 pooled values); it resets the header words when hdr is set.
hipError_t prepass(const uint16_t* q16, const uint16_t* k16, const uint16_t* v16, float* kpool, float* vmean,
                   int BH, int N, int d, bool row_corr, unsigned char* wsb, unsigned* hdr, hipStream_t s) {
  const WsLayout w = ws_layout(BH, N, d);
  const int Nk = (N + 63) / 64;
  sol::PoolSet set;
  set.planes.kh = reinterpret_cast<uint16_t*>(wsb + w.kh);
  set.planes.km = reinterpret_cast<uint16_t*>(wsb + w.km);
  set.planes.kl = reinterpret_cast<uint16_t*>(wsb + w.kl);
  set.planes.vt = reinterpret_cast<uint16_t*>(wsb + w.vt);
  set.planes.vrow = row_corr ? reinterpret_cast<uint16_t*>(wsb + w.vbar16) : nullptr;
  set.planes.kpool = kpool;
  set.planes.vmean = vmean;
  set.planes.Nkp = padded_blocks(Nk);
  set.src[0] = q16;
  set.dst[0] = reinterpret_cast<float*>(wsb + w.qpool);
  set.n = 1;
  if (k16 == nullptr) {
    set.role[0] = sol::kRoleKeysFromPool | sol::kRoleValuesFromPool;
  } else {
    set.src[1] = k16;
    set.dst[1] = kpool;
    set.role[1] = sol::kRoleKeys;
    set.src[2] = v16;
    set.dst[2] = vmean;
    set.role[2] = sol::kRoleValues;
    set.n = 3;
  }
  return sol::launch_pool(set, BH, N, Nk, d, hdr, s);
}

int forward_impl(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                 int Bq, int Bk, const sol_attn_route& route, unsigned flags, sol_attn_stats* stats, float* kpool,
                 float* vmean, void* ws, size_t ws_bytes, void* stream, uint32_t* bitmap) {
  const int rc = check_forward(q, k, v, out, B, H, N, d, Bq, Bk, route, flags, stats, kpool, vmean, ws, ws_bytes);
  if (rc != SOL_OK) return rc;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int BH = B * H;
  const int Nq = (N + Bq - 1) / Bq, Nk = (N + Bk - 1) / Bk;
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const uint16_t* k16 = static_cast<const uint16_t*>(k);
  const uint16_t* v16 = static_cast<const uint16_t*>(v);
  const WsLayout w = ws_layout(BH, N, d);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  const int group = group_of(flags, BH, Nq, route);
  const int nitems = sol::forward_items(BH, Nq, group);

  const unsigned* units = nullptr;
  hipError_t e = hipSuccess;
  // the pooling pre-pass (unless the workspace holds it already); the header
  // words are reset by it or, after sol_attn_prepare, by a reset kernel,
  // except where a plan left them clean
  float* qpool = reinterpret_cast<float*>(wsb + w.qpool);
  uint16_t* kh = reinterpret_cast<uint16_t*>(wsb + w.kh);
  uint16_t* km = reinterpret_cast<uint16_t*>(wsb + w.km);
  uint16_t* kl = reinterpret_cast<uint16_t*>(wsb + w.kl);
  uint16_t* vt = reinterpret_cast<uint16_t*>(wsb + w.vt);
  uint16_t* vbar16 = reinterpret_cast<uint16_t*>(wsb + w.vbar16);
  const int Nkp = padded_blocks(Nk);
  unsigned* hdr = (flags & SOL_F_PLANNED) ? nullptr : static_cast<unsigned*>(ws);
  if (flags & SOL_F_PREPARED) {
    if (hdr) e = sol::launch_reset(hdr, s);
  } else {
    const bool pooled = flags & SOL_F_POOLED;
    e = prepass(q16, pooled ? nullptr : k16, pooled ? nullptr : v16, kpool, vmean, BH, N, d,
                flags & SOL_F_ROW_CORRECTION, wsb, hdr, s);
  }
  if (e != hipSuccess) return SOL_EHIP;
  if (flags & SOL_F_PLANNED) {
    // the workspace holds a valid order from sol_attn_plan(), as a previous call left it
    units = reinterpret_cast<const unsigned*>(wsb + w.units);
  } else {
    // plan the order of the work where that was measured to pay (elsewhere
    // the items go in sequence; the order never changes the result)
    if (e == hipSuccess && plan_by_default(route, BH, Nq, nitems, group)) {
      bool ordered = false;
      e = plan_impl(q16, kpool, BH, N, d, route.tau, ws, s, &ordered);
      units = reinterpret_cast<const unsigned*>(wsb + w.units);
    }
  }
  if (e != hipSuccess) return SOL_EHIP;
  float* kstats = reinterpret_cast<float*>(wsb + w.kstats);
  if (route.rule == SOL_ROUTE_GAUSS_DIAG) {
    e = sol::launch_kstats(kpool, kstats, BH, Nk, d, s);
    if (e != hipSuccess) return SOL_EHIP;
  }
  float* kmom = reinterpret_cast<float*>(wsb + w.kmom);
  if (route.rule == SOL_ROUTE_GAUSS) {
    e = sol::launch_kmom(kpool, kmom, BH, Nk, d, s);
    if (e != hipSuccess) return SOL_EHIP;
  }

  sol::FwdParams p;
  p.q = q16;
  p.k = k16;
  p.v = v16;
  p.out = out;
  p.kpool = kpool;
  p.vmean = vmean;
  p.units = units;
  p.plan_items = reinterpret_cast<const unsigned*>(wsb + w.plan);
  p.hdr = static_cast<unsigned*>(ws);
  p.stats = stats;
  p.bitmap = bitmap;
  p.N = N;
  p.Nq = Nq;
  p.Nk = Nk;
  p.nitems = nitems;
  p.nwords = (Nk + 31) / 32;
  p.group = group;
  p.ngroups = (Nq + group - 1) / group;
  p.route_only = 0;
  p.static_grid = 0;
  // without a plan, every block kept (tau = +inf): each queue's last items
  // (one per workgroup of its XCD) go out pair by pair; the routing pass is
  // then a small part of an item
  p.split_n = route.rule == SOL_ROUTE_ROWMAX && isinf(route.tau) ? std::max(1, device_cus() / 4) : 0;
  p.kmom = kmom;
  p.rule = route.rule;
  p.tau = route.rule == SOL_ROUTE_ROWMAX ? route.tau : 0.f;
  p.beta = route.rule != SOL_ROUTE_ROWMAX ? route.beta : 0.f;
  p.kstats = kstats;
  p.sink_lo = route.sink_count > 0 ? route.sink_first : 0;
  p.sink_hi = route.sink_count > 0 ? route.sink_first + route.sink_count : 0;
  p.proxy_scale = (float)(1.0 / sqrt((double)d));
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  p.exact_only = (flags & SOL_F_EXACT_ONLY) ? 1 : 0;
  p.row_corr = (flags & SOL_F_ROW_CORRECTION) ? 1 : 0;
  p.out_bf16 = (flags & SOL_F_OUT_BF16) ? 1 : 0;
  p.khi16 = kh;
  p.klo16 = km;
  p.klo2 = kl;
  p.vt = vt;
  p.Nkp = Nkp;
  p.vbar16 = vbar16;
  p.qpool = qpool;
  e = sol::launch_forward(p, d, s);
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

// Workspace of the mask builders: top-k / top-p use [pooled queries | map];
// the threshold router uses [three bf16 planes of the pooled keys | pooled
// queries].
struct MaskWs {
  size_t map, total;
};

MaskWs mask_ws(int BH, int N, int d) {
  const size_t Nq = (size_t)(N + 63) / 64;
  MaskWs w;
  w.map = round_up((size_t)BH * Nq * (size_t)d * 4, 256);
  const size_t planes = 3 * round_up((size_t)BH * padded_blocks((int)Nq) * (size_t)d * 2, 256) +
                        round_up((size_t)BH * Nq * (size_t)d * 4, 256);
  w.total = std::max(round_up(w.map + (size_t)BH * Nq * Nq * 4, 256), planes);
  return w;
}

int check_mask(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, const uint32_t* bitmap) {
  if (!q || !kpool || !bitmap) return SOL_EINVAL;
  if (!aligned(q, 16) || !aligned(kpool, 16) || !aligned(bitmap, 4)) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, Bq, Bk);
  if (rc != SOL_OK) return rc;
  if ((long long)B * H > kMaxGridHeads) return SOL_EUNSUPPORTED;
  return SOL_OK;
}

int sorted_mask(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, int topk, float topp,
                int mode, uint32_t* bitmap, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_mask(q, kpool, B, H, N, d, Bq, Bk, bitmap);
  if (rc != SOL_OK) return rc;
  if (mode == 1 && isnan(topp)) return SOL_EINVAL;
  if (!ws || !aligned(ws, 256)) return SOL_EINVAL;
  const int BH = B * H, Nq = (N + 63) / 64, Nk = Nq;
  const MaskWs w = mask_ws(BH, N, d);
  if (ws_bytes < w.total) return SOL_EWORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float* qpool = reinterpret_cast<float*>(wsb);
  float* map = reinterpret_cast<float*>(wsb + w.map);
  sol::PoolSet set;
  set.src[0] = static_cast<const uint16_t*>(q);
  set.dst[0] = qpool;
  set.n = 1;
  hipError_t e = sol::launch_pool(set, BH, N, Nk, d, nullptr, s);
  if (e == hipSuccess) e = sol::launch_proxy_map(qpool, kpool, map, BH, Nq, Nk, d, (float)(1.0 / sqrt((double)d)), s);
  if (e == hipSuccess) e = sol::launch_sort_mask(map, bitmap, BH, Nq, Nk, topk, topp, mode, s);
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

}  // namespace

extern "C" {

size_t sol_attn_mask_workspace_bytes(int B, int H, int N, int d, int Bq, int Bk) {
  if (check_sizes(B, H, N, d, Bq, Bk) != SOL_OK || (long long)B * H > kMaxGridHeads) return 0;
  return mask_ws(B * H, N, d).total;
}

int sol_attn_mask_threshold(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk,
                            const sol_attn_route* route, uint32_t* kept_bitmap, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int rc = check_mask(q, kpool, B, H, N, d, Bq, Bk, kept_bitmap);
  if (rc != SOL_OK) return rc;
  if (!route || check_route(*route, N, Bk) != SOL_OK) return SOL_EINVAL;
  // the Gaussian rules take their statistics from the forward's workspace
  if (route->rule != SOL_ROUTE_ROWMAX) return SOL_EUNSUPPORTED;
  if (!workspace || !aligned(workspace, 256)) return SOL_EINVAL;
  const int BH = B * H, Nq = (N + 63) / 64;
  if (workspace_bytes < mask_ws(BH, N, d).total) return SOL_EWORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the score operands (the pooled keys in three bf16 parts, the pooled
  // queries), as the forward makes them
  const size_t plane = round_up((size_t)BH * padded_blocks(Nq) * (size_t)d * 2, 256);
  uint16_t* kh = static_cast<uint16_t*>(workspace);
  uint16_t* km = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(workspace) + plane);
  uint16_t* kl = reinterpret_cast<uint16_t*>(static_cast<unsigned char*>(workspace) + 2 * plane);
  float* qpool = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + 3 * plane);
  sol::PoolSet set;
  set.src[0] = static_cast<const uint16_t*>(q);
  set.dst[0] = qpool;
  set.role[0] = sol::kRoleKeysFromPool;
  set.n = 1;
  set.planes.kh = kh;
  set.planes.km = km;
  set.planes.kl = kl;
  set.planes.kpool = kpool;
  set.planes.Nkp = padded_blocks(Nq);
  hipError_t e = sol::launch_pool(set, BH, N, Nq, d, nullptr, s);
  if (e != hipSuccess) return SOL_EHIP;
  // the forward's own fused kernel, stopped after its routing: one workgroup
  // per item, no work queues, no correction sums; only the bitmap is written
  sol::FwdParams p = {};
  p.q = static_cast<const uint16_t*>(q);
  p.kpool = kpool;
  p.vmean = kpool;  // not read: no correction sums are formed
  p.khi16 = kh;
  p.klo16 = km;
  p.klo2 = kl;
  p.Nkp = padded_blocks(Nq);
  p.qpool = qpool;
  p.bitmap = kept_bitmap;
  p.N = N;
  p.Nq = Nq;
  p.Nk = Nq;
  p.nwords = (Nq + 31) / 32;
  // (at most four blocks per item: the routing-only kernel then fits four
  // workgroups per CU without spilling)
  p.group = std::min(auto_group(BH, Nq, *route), 4);
  p.ngroups = (Nq + p.group - 1) / p.group;
  p.nitems = sol::forward_items(BH, Nq, p.group);
  p.route_only = 1;
  p.static_grid = 1;
  p.rule = SOL_ROUTE_ROWMAX;
  p.tau = route->tau;
  p.sink_lo = route->sink_count > 0 ? route->sink_first : 0;
  p.sink_hi = route->sink_count > 0 ? route->sink_first + route->sink_count : 0;
  p.proxy_scale = (float)(1.0 / sqrt((double)d));
  p.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
  p.exact_only = 1;
  e = sol::launch_forward(p, d, s);
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

int sol_attn_mask_topk(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, int k,
                       uint32_t* kept_bitmap, void* workspace, size_t workspace_bytes, void* stream) {
  return sorted_mask(q, kpool, B, H, N, d, Bq, Bk, k, 0.f, 0, kept_bitmap, workspace, workspace_bytes, stream);
}

int sol_attn_mask_topp(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, float p,
                       uint32_t* kept_bitmap, void* workspace, size_t workspace_bytes, void* stream) {
  return sorted_mask(q, kpool, B, H, N, d, Bq, Bk, 0, p, 1, kept_bitmap, workspace, workspace_bytes, stream);
}

size_t sol_attn_workspace_bytes(int B, int H, int N, int d, int Bq, int Bk) {
  if (check_sizes(B, H, N, d, Bq, Bk) != SOL_OK) return 0;
  return ws_layout(B * H, N, d).total;
}

int sol_attn_pool(const void* k, const void* v, float* kpool, float* vmean, int B, int H, int N, int d,
                  int Bk, void* stream) {
  if (!k || !v || !kpool || !vmean) return SOL_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kpool, 16) || !aligned(vmean, 16)) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, 64, Bk);
  if (rc != SOL_OK) return rc;
  const int Nk = (N + Bk - 1) / Bk;
  sol::PoolSet set;
  set.src[0] = static_cast<const uint16_t*>(k);
  set.dst[0] = kpool;
  set.src[1] = static_cast<const uint16_t*>(v);
  set.dst[1] = vmean;
  set.n = 2;
  const hipError_t e = sol::launch_pool(set, B * H, N, Nk, d, nullptr, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

int sol_attn_plan(const void* q, const float* kpool, int B, int H, int N, int d, int Bq, int Bk, float tau,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !kpool || !workspace) return SOL_EINVAL;
  if (!aligned(q, 16) || !aligned(kpool, 16) || !aligned(workspace, 256)) return SOL_EINVAL;
  if (check_tau(tau) != SOL_OK) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, Bq, Bk);
  if (rc != SOL_OK) return rc;
  if (workspace_bytes < sol_attn_workspace_bytes(B, H, N, d, Bq, Bk)) return SOL_EWORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = sol::launch_reset(static_cast<unsigned*>(workspace), s);
  bool ordered = false;
  if (e == hipSuccess) e = plan_impl(static_cast<const uint16_t*>(q), kpool, B * H, N, d, tau, workspace, s, &ordered);
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

int sol_attn_prepare(const void* q, const float* kpool, const float* vmean, int B, int H, int N, int d, int Bq,
                     int Bk, unsigned flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !kpool || !vmean || !workspace) return SOL_EINVAL;
  if (!aligned(q, 16) || !aligned(kpool, 16) || !aligned(vmean, 16) || !aligned(workspace, 256)) return SOL_EINVAL;
  if (flags & ~(unsigned)SOL_F_ROW_CORRECTION) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, Bq, Bk);
  if (rc != SOL_OK) return rc;
  if (workspace_bytes < sol_attn_workspace_bytes(B, H, N, d, Bq, Bk)) return SOL_EWORKSPACE;
  const hipError_t e = prepass(static_cast<const uint16_t*>(q), nullptr, nullptr, const_cast<float*>(kpool),
                               const_cast<float*>(vmean), B * H, N, d, flags & SOL_F_ROW_CORRECTION,
                               static_cast<unsigned char*>(workspace), nullptr, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

int sol_attn_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                     int Bq, int Bk, float tau, unsigned flags, sol_attn_stats* stats, float* kpool,
                     float* vmean, void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(q, k, v, out, B, H, N, d, Bq, Bk, rowmax_route(tau), flags, stats, kpool, vmean, workspace,
                      workspace_bytes, stream, nullptr);
}

int sol_attn_forward_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                        int Bq, int Bk, const sol_attn_route* route, unsigned flags, sol_attn_stats* stats,
                        float* kpool, float* vmean, void* workspace, size_t workspace_bytes, void* stream,
                        uint32_t* kept_bitmap) {
  if (!route) return SOL_EINVAL;
  if (kept_bitmap && !aligned(kept_bitmap, 4)) return SOL_EINVAL;
  return forward_impl(q, k, v, out, B, H, N, d, Bq, Bk, *route, flags, stats, kpool, vmean, workspace,
                      workspace_bytes, stream, kept_bitmap);
}

int sol_attn_forward_debug(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                           int d, int Bq, int Bk, float tau, unsigned flags, sol_attn_stats* stats,
                           float* kpool, float* vmean, void* workspace, size_t workspace_bytes,
                           void* stream, uint32_t* kept_bitmap) {
  if (!kept_bitmap || !aligned(kept_bitmap, 4)) return SOL_EINVAL;
  return forward_impl(q, k, v, out, B, H, N, d, Bq, Bk, rowmax_route(tau), flags, stats, kpool, vmean, workspace,
                      workspace_bytes, stream, kept_bitmap);
}

int sol_attn_forward_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int N, int d,
                             int Bq, int Bk, const sol_attn_route* route, unsigned flags, sol_attn_stats* stats,
                             void* stream, uint32_t* kept_bitmap) {
  if (!route) return SOL_EINVAL;
  if (kept_bitmap && !aligned(kept_bitmap, 4)) return SOL_EINVAL;
  // the pooled buffers and the plan live in the shared scratch array, which
  // the previous call on this GPU may have overwritten: always pool afresh
  if (flags & (SOL_F_POOLED | SOL_F_PLANNED | SOL_F_PREPARED)) return SOL_EINVAL;
  const int rc = check_args(q, k, v, out, B, H, N, d, Bq, Bk, *route, flags, stats);
  if (rc != SOL_OK) return rc;
  // scratch layout: [workspace | kpool | vmean], each 256-byte aligned
  const size_t ws = sol_attn_workspace_bytes(B, H, N, d, Bq, Bk);
  const size_t pooled = round_up((size_t)B * H * (size_t)((N + Bk - 1) / Bk) * (size_t)d * 4, 256);
  if (ws + 2 * pooled > (size_t)SOL_ATTN_SCRATCH_BYTES) return SOL_ESCRATCH;
  void* base = nullptr;
  const int rc3 = scratch_base(&base);
  if (rc3 != SOL_OK) return rc3;
  unsigned char* b = static_cast<unsigned char*>(base);
  return forward_impl(q, k, v, out, B, H, N, d, Bq, Bk, *route, flags, stats, reinterpret_cast<float*>(b + ws),
                      reinterpret_cast<float*>(b + ws + pooled), b, ws, stream, kept_bitmap);
}

const char* sol_attn_strerror(int code) {
  switch (code) {
    case SOL_OK: return "success";
    case SOL_EINVAL:
      return "invalid argument (null/misaligned pointer, size <= 0, tau NaN or negative, beta not finite, "
             "unknown rule, sink range out of bounds, unknown or inconsistent flags, exact-only under a "
             "Gaussian rule without sinks)";
    case SOL_EUNSUPPORTED: return "unsupported configuration (d must be 64 or 128, Bq = Bk = 64, N <= SOL_ATTN_MAX_N)";
    case SOL_EWORKSPACE: return "workspace smaller than sol_attn_workspace_bytes()";
    case SOL_EHIP: return "HIP runtime error during launch";
    case SOL_ESCRATCH:
      return "problem too large for sol_attn_forward_noalloc (needs more than SOL_ATTN_SCRATCH_BYTES of scratch)";
    default: return "unknown error code";
  }
}

}  // extern "C"
