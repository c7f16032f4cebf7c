// C ABI entry points: argument validation (entirely on the host, before any
// launch), then kernel launches on the caller's stream.
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "sol_attn.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: [header words | item costs | item order | pooled-key copies and
// statistics of the optional modes].
struct WsLayout {
  size_t cost, perm, khi16, klo16, vbar16, kstats, total;
};

WsLayout ws_layout(int BH, int N, int d) {
  const size_t Nq = (size_t)(N + 63) / 64;
  const size_t items = (size_t)sol::forward_items(BH, (int)Nq);
  WsLayout w;
  w.cost = sol::kHdrWords * 4;
  w.perm = round_up(w.cost + 4 * items, 256);
  w.khi16 = round_up(w.perm + 4 * items, 256);
  w.klo16 = round_up(w.khi16 + (size_t)BH * Nq * (size_t)d * 2, 256);
  w.vbar16 = round_up(w.klo16 + (size_t)BH * Nq * (size_t)d * 2, 256);
  w.kstats = round_up(w.vbar16 + (size_t)BH * Nq * (size_t)d * 2, 256);
  w.total = round_up(w.kstats + (size_t)BH * 2 * (size_t)d * 4, 256);
  return w;
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

bool plan_by_default(const sol_attn_route& r, int BH, int Nq, int nitems) {
  return r.rule == SOL_ROUTE_ROWMAX && r.tau >= kPlanMinTau && use_order(r.tau, nitems) &&
         nitems <= kPlanMaxItems && (long long)BH * Nq * Nq >= kPlanMinPairs && BH <= kMaxGridHeads;
}

int check_sizes(int B, int H, int N, int d, int Bq, int Bk) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || Bq <= 0 || Bk <= 0) return SOL_EINVAL;
  if (d != 64 && d != 128) return SOL_EUNSUPPORTED;
  if (Bq != 64 || Bk != 64) return SOL_EUNSUPPORTED;
  if (N > SOL_ATTN_MAX_N) return SOL_EUNSUPPORTED;
  const long long nq = (N + 63) / 64;
  if (nq > sol::forward_max_blocks(d)) return SOL_EUNSUPPORTED;
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
// order, which every later planned forward may still read.
hipError_t plan_impl(const uint16_t* q, const float* kpool, int BH, int N, int d, float tau, void* ws, hipStream_t s,
                     bool* ordered) {
  const WsLayout w = ws_layout(BH, N, d);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  const int Nq = (N + 63) / 64, Nk = Nq;
  unsigned* perm = reinterpret_cast<unsigned*>(wsb + w.perm);
  const int nitems = sol::forward_items(BH, Nq);
  *ordered = use_order(tau, nitems) && BH <= kMaxGridHeads;
  if (*ordered)
    return sol::launch_plan(q, kpool, reinterpret_cast<unsigned*>(wsb + w.cost), perm, BH, N, Nq, Nk, d, tau,
                            (float)(1.0 / sqrt((double)d)), s);
  return sol::launch_identity_order(perm, nitems, s);
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

int check_forward(const void* q, const void* k, const void* v, const void* out, int B, int H, int N,
                  int d, int Bq, int Bk, const sol_attn_route& route, unsigned flags, const sol_attn_stats* stats,
                  const float* kpool, const float* vmean, const void* ws, size_t ws_bytes) {
  if (!q || !k || !v || !out || !kpool || !vmean || !ws) return SOL_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(kpool, 16) || !aligned(vmean, 16) || !aligned(ws, 256) || !aligned(stats, 8))
    return SOL_EINVAL;
  if (check_route(route, N, Bk) != SOL_OK) return SOL_EINVAL;
  if (flags & ~(unsigned)(SOL_F_POOLED | SOL_F_EXACT_ONLY | SOL_F_PLANNED | SOL_F_ROW_CORRECTION | SOL_F_OUT_BF16))
    return SOL_EINVAL;
  if ((flags & SOL_F_EXACT_ONLY) && (flags & SOL_F_ROW_CORRECTION)) return SOL_EINVAL;
  if ((flags & SOL_F_PLANNED) && !(flags & SOL_F_POOLED)) return SOL_EINVAL;
  const int rc = check_sizes(B, H, N, d, Bq, Bk);
  if (rc != SOL_OK) return rc;
  if (ws_bytes < sol_attn_workspace_bytes(B, H, N, d, Bq, Bk)) return SOL_EWORKSPACE;
  return SOL_OK;
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
  const int nitems = sol::forward_items(BH, Nq);

  const unsigned* perm = nullptr;
  hipError_t e = hipSuccess;
  if (flags & SOL_F_PLANNED) {
    // the workspace holds a valid order from sol_attn_plan(), as a previous call left it
    perm = reinterpret_cast<const unsigned*>(wsb + w.perm);
  } else {
    if (flags & SOL_F_POOLED) {
      e = sol::launch_reset(static_cast<unsigned*>(ws), s);
    } else {
      sol::PoolSet set;
      set.src[0] = k16;
      set.dst[0] = kpool;
      set.src[1] = v16;
      set.dst[1] = vmean;
      set.n = 2;
      e = sol::launch_pool(set, BH, N, Nk, d, static_cast<unsigned*>(ws), s);
    }
    // plan the order of the work where that was measured to pay (elsewhere
    // the items go in sequence; the order never changes the result)
    if (e == hipSuccess && plan_by_default(route, BH, Nq, nitems)) {
      bool ordered = false;
      e = plan_impl(q16, kpool, BH, N, d, route.tau, ws, s, &ordered);
      perm = reinterpret_cast<const unsigned*>(wsb + w.perm);
    }
  }
  if (e != hipSuccess) return SOL_EHIP;
  uint16_t* khi16 = reinterpret_cast<uint16_t*>(wsb + w.khi16);
  uint16_t* klo16 = reinterpret_cast<uint16_t*>(wsb + w.klo16);
  uint16_t* vbar16 = reinterpret_cast<uint16_t*>(wsb + w.vbar16);
  if (flags & SOL_F_ROW_CORRECTION) {
    e = sol::launch_to_bf16(kpool, khi16, klo16, vmean, vbar16, (size_t)BH * Nk * d, s);
    if (e != hipSuccess) return SOL_EHIP;
  }
  float* kstats = reinterpret_cast<float*>(wsb + w.kstats);
  if (route.rule == SOL_ROUTE_GAUSS_DIAG) {
    e = sol::launch_kstats(kpool, kstats, BH, Nk, d, s);
    if (e != hipSuccess) return SOL_EHIP;
  }

  sol::FwdParams p;
  p.q = q16;
  p.k = k16;
  p.v = v16;
  p.out = out;
  p.kpool = kpool;
  p.vmean = vmean;
  p.perm = perm;
  p.hdr = static_cast<unsigned*>(ws);
  p.stats = stats;
  p.bitmap = bitmap;
  p.N = N;
  p.Nq = Nq;
  p.Nk = Nk;
  p.nitems = nitems;
  p.nwords = (Nk + 31) / 32;
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
  p.khi16 = khi16;
  p.klo16 = klo16;
  p.vbar16 = vbar16;
  e = sol::launch_forward(p, d, s);
  return e == hipSuccess ? SOL_OK : SOL_EHIP;
}

// Workspace of the top-k / top-p mask builders: pooled queries, then the map.
struct MaskWs {
  size_t map, total;
};

MaskWs mask_ws(int BH, int N, int d) {
  const size_t Nq = (size_t)(N + 63) / 64;
  MaskWs w;
  w.map = round_up((size_t)BH * Nq * (size_t)d * 4, 256);
  w.total = round_up(w.map + (size_t)BH * Nq * Nq * 4, 256);
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
                            const sol_attn_route* route, uint32_t* kept_bitmap, void* stream) {
  int rc = check_mask(q, kpool, B, H, N, d, Bq, Bk, kept_bitmap);
  if (rc != SOL_OK) return rc;
  if (!route || check_route(*route, N, Bk) != SOL_OK) return SOL_EINVAL;
  if (route->rule == SOL_ROUTE_GAUSS_DIAG) return SOL_EUNSUPPORTED;
  sol::MaskParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.kpool = kpool;
  p.bitmap = kept_bitmap;
  p.N = N;
  p.Nq = (N + 63) / 64;
  p.Nk = p.Nq;
  p.nwords = (p.Nk + 31) / 32;
  p.rule = route->rule;
  p.tau = route->rule == SOL_ROUTE_ROWMAX ? route->tau : 0.f;
  p.beta = route->rule == SOL_ROUTE_GAUSS ? route->beta : 0.f;
  p.proxy_scale = (float)(1.0 / sqrt((double)d));
  p.sink_lo = route->sink_count > 0 ? route->sink_first : 0;
  p.sink_hi = route->sink_count > 0 ? route->sink_first + route->sink_count : 0;
  const hipError_t e = sol::launch_mask_threshold(p, d, B * H, reinterpret_cast<hipStream_t>(stream));
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

const char* sol_attn_strerror(int code) {
  switch (code) {
    case SOL_OK: return "success";
    case SOL_EINVAL:
      return "invalid argument (null/misaligned pointer, size <= 0, tau NaN or negative, beta not finite, "
             "unknown rule, sink range out of bounds, unknown or inconsistent flags)";
    case SOL_EUNSUPPORTED: return "unsupported configuration (d must be 64 or 128, Bq = Bk = 64, N <= SOL_ATTN_MAX_N)";
    case SOL_EWORKSPACE: return "workspace smaller than sol_attn_workspace_bytes()";
    case SOL_EHIP: return "HIP runtime error during launch";
    default: return "unknown error code";
  }
}

}  // extern "C"
