// C ABI of the device entry points: validation (complete before any HIP
// call), slot-table construction, workspace layout, launch and timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "sfa_device.h"
#include "sfa_internal.h"
#include "sfa_launch.h"

namespace sfa {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate_problem(const sfa_attn* a, Problem* p) {
  if (!a) return fail(SFA_ERR_ARG, "problem is NULL");
  if (a->batch < 0 || a->seqlen < 0) return fail(SFA_ERR_ARG, "batch and seqlen must be >= 0");
  if (a->hq < 1 || a->hkv < 1 || a->hq % a->hkv)
    return fail(SFA_ERR_ARG, "hq must be a positive multiple of hkv");
  const int G = a->hq / a->hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SFA_ERR_UNSUPPORTED, "group size hq/hkv = %d not in {1,2,4,8}", G);
  if (a->head_dim != 16 && a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128)
    return fail(SFA_ERR_UNSUPPORTED, "head_dim %d not in {16,32,64,128}", a->head_dim);
  // fp32 rows of 128 dims would put a stage's V rows beyond the reach of an
  // LDS instruction's offset from its K rows; only bf16 tensors are built there.
  if (a->head_dim == 128 && a->dtype == SFA_F32)
    return fail(SFA_ERR_UNSUPPORTED, "head_dim 128 is built for bf16 tensors only");
  if (a->head_dim / G < 2) return fail(SFA_ERR_UNSUPPORTED, "head_dim / group < 2");
  if (a->dtype != SFA_F32 && a->dtype != SFA_BF16) return fail(SFA_ERR_ARG, "unknown dtype %d", a->dtype);
  if (a->window < 0) return fail(SFA_ERR_ARG, "window must be >= 0");
  if (a->n_off < 0 || a->n_off > SFA_MAX_OFFSETS)
    return fail(SFA_ERR_UNSUPPORTED, "n_off %d not in [0, %d]", a->n_off, SFA_MAX_OFFSETS);
  if (int64_t(a->window) + 1 + a->n_off > SFA_MAX_SLOTS)
    return fail(SFA_ERR_UNSUPPORTED, "window + 1 + n_off exceeds %d slots", SFA_MAX_SLOTS);
  if (a->flags & ~(SFA_FLAG_INTERP_KERNEL | SFA_FLAG_SIGNED_OFFSETS))
    return fail(SFA_ERR_ARG, "unknown flags 0x%x", unsigned(a->flags));
  const int32_t lo_min = (a->flags & SFA_FLAG_SIGNED_OFFSETS) ? -(1 << 30) + 1 : 0;
  if (!std::isfinite(a->scale) || a->scale < 0.f) return fail(SFA_ERR_ARG, "scale must be finite and >= 0");
  if (a->n_off > 0 && (!a->off_lo || !a->off_frac)) return fail(SFA_ERR_ARG, "offset arrays are NULL");
  for (int k = 0; k < a->n_off; ++k) {
    if (a->off_lo[k] < lo_min || a->off_lo[k] >= (1 << 30))
      return fail(SFA_ERR_ARG, "off_lo[%d] = %d out of range%s", k, a->off_lo[k],
                  a->off_lo[k] < 0 ? " (negative offsets need SFA_FLAG_SIGNED_OFFSETS)" : "");
    const float f = a->off_frac[k];
    if (!(f >= 0.f && f < 1.f)) return fail(SFA_ERR_ARG, "off_frac[%d] not in [0,1)", k);
  }
  if (a->rope && (reinterpret_cast<uintptr_t>(a->rope) & 7u)) return fail(SFA_ERR_ARG, "rope table not 8-byte aligned");
  const int64_t elems = int64_t(a->batch) * a->seqlen * a->hq * a->head_dim;
  if (elems >= (int64_t(1) << 40)) return fail(SFA_ERR_UNSUPPORTED, "tensor too large");
  p->B = a->batch;
  p->n = a->seqlen;
  p->hq = a->hq;
  p->hkv = a->hkv;
  p->D = a->head_dim;
  p->G = G;
  p->dtype = a->dtype;
  p->window = a->window;
  p->n_off = a->n_off;
  p->flags = a->flags;
  p->scale = a->scale > 0.f ? a->scale : float(1.0 / std::sqrt(double(a->head_dim)));
  p->rope = a->rope;
  return SFA_OK;
}

int build_slots(const sfa_attn* a, SlotTable* t, bool merge) {
  struct S {
    int32_t lo;
    float frac;
    int32_t rung;
  };
  std::vector<S> v;
  v.reserve(size_t(a->window) + 1 + size_t(a->n_off));
  for (int s = 0; s <= a->window; ++s) v.push_back({s, 0.f, -1});
  for (int k = 0; k < a->n_off; ++k) v.push_back({a->off_lo[k], a->off_frac[k], int32_t(k)});
  std::stable_sort(v.begin(), v.end(), [](const S& x, const S& y) { return x.lo < y.lo; });
  std::memset(t, 0, sizeof(*t));
  t->n_rungs = a->n_off;
  int c = 0;
  for (size_t s = 0; s < v.size(); ++s) {
    if (merge && c > 0 && t->s[c - 1].lo == v[s].lo && t->s[c - 1].frac == v[s].frac) {
      t->s[c - 1].mult += 1.f;
      t->s[c - 1].rung = -1;
      continue;
    }
    t->s[c].lo = v[s].lo;
    // Kernels test frac != 0 on its bit pattern (a scalar compare), so a
    // zero fraction is stored as +0.
    t->s[c].frac = v[s].frac == 0.f ? 0.f : v[s].frac;
    t->s[c].mult = 1.f;
    t->s[c].rung = v[s].rung;
    ++c;
  }
  t->count = c;
  return SFA_OK;
}

// ----------------------------------------------------------------- timing

namespace {
struct Pending {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // record only this kernel's launches when not empty
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;  // recycled events: no creation per launch
std::map<std::string, std::pair<double, int64_t>> g_totals;

hipEvent_t take_event() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

thread_local ProfileScope* tl_scope = nullptr;

ProfileScope* active_profile_scope() { return tl_scope; }

ProfileScope::ProfileScope(const char* nm, void* st) : name(nm), stream(st), ev0(nullptr), ev1(nullptr), launches(0) {
  if (!g_prof_on || !nm) return;  // a null name records nothing
  if (!g_prof_only.empty() && g_prof_only != nm) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (a) g_free.push_back(a);
    if (b) g_free.push_back(b);
    return;
  }
  ev0 = a;
  ev1 = b;
  tl_scope = this;
}

ProfileScope::~ProfileScope() {
  if (!ev0) return;
  tl_scope = nullptr;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  bool ok = launches > 0;  // the first launch took the pair
  if (launches > 1) ok = hipEventRecord(static_cast<hipEvent_t>(ev1), st) == hipSuccess;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!ok) {
    g_free.push_back(static_cast<hipEvent_t>(ev0));
    g_free.push_back(static_cast<hipEvent_t>(ev1));
    return;
  }
  g_pending.push_back({name, static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1)});
}

static void drain_pending() {
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      auto& t = g_totals[p.name];
      t.first += ms;
      t.second += 1;
    }
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
}

static int hip_status(int err, const char* what) {
  if (err != 0)
    return fail(SFA_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
  return SFA_OK;
}

}  // namespace sfa

using namespace sfa;

extern "C" int sfa_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return SFA_OK;
}

extern "C" int sfa_profile_select(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = kernel ? kernel : "";
  return SFA_OK;
}

extern "C" int sfa_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending();
  g_totals.clear();
  return SFA_OK;
}

extern "C" int sfa_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel) return fail(SFA_ERR_ARG, "sfa_profile_read: kernel is NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending();
  auto it = g_totals.find(kernel);
  if (total_ms) *total_ms = it == g_totals.end() ? 0.0 : it->second.first;
  if (launches) *launches = it == g_totals.end() ? 0 : it->second.second;
  return SFA_OK;
}

// ------------------------------------------------------------ range scan

namespace {

// Largest |x| of count elements, as IEEE bits (NaN above +inf above every
// finite value, so the bit order is the magnitude order with non-finite
// values on top): every thread reads 8 elements (16 bytes of bf16, two
// float4 of fp32) per grid-stride iteration, the wave takes the maximum of
// its lanes and one lane per wave folds it into *result with an atomic max.
template <typename T>
__global__ __launch_bounds__(256) void absmax_kernel(const T* __restrict__ x, int64_t count,
                                                     unsigned* __restrict__ result) {
  unsigned m = 0;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x * 8;
  for (int64_t i0 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8; i0 < count; i0 += stride) {
    float v[8];
    if (i0 + 8 <= count) {
      load_vec<8>(x + i0, v);
    } else {
      for (int u = 0; u < 8; ++u) v[u] = i0 + u < count ? load1(x + i0 + u) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) m = max(m, __float_as_uint(v[u]) & 0x7fffffffu);
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = max(m, unsigned(__shfl_xor(int(m), s)));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(result, m);
}

}  // namespace

// ------------------------------------------------------------ entry points

extern "C" int sfa_absmax(const void* x, int64_t count, int dtype, uint32_t* result, void* stream) {
  clear_error();
  if (count < 0) return fail(SFA_ERR_ARG, "sfa_absmax: count must be >= 0");
  if (dtype != SFA_F32 && dtype != SFA_BF16) return fail(SFA_ERR_ARG, "sfa_absmax: unknown dtype %d", dtype);
  if (count == 0) return SFA_OK;
  if (!x || !result) return fail(SFA_ERR_ARG, "sfa_absmax: NULL pointer");
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(result) & 3u))
    return fail(SFA_ERR_ARG, "sfa_absmax: x must be 16-byte aligned, result 4-byte aligned");
  const int64_t per_block = 256 * 8;
  const int blocks = int(std::min<int64_t>((count + per_block - 1) / per_block, 2048));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SFA_BF16)
    SFA_LAUNCH(absmax_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, static_cast<const bf16_t*>(x), count,
                       reinterpret_cast<unsigned*>(result));
  else
    SFA_LAUNCH(absmax_kernel<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float*>(x), count,
                       reinterpret_cast<unsigned*>(result));
  return hip_status(int(hipGetLastError()), "sfa_absmax launch");
}

extern "C" int sfa_fwd(const sfa_attn* a, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* stream) {
  clear_error();
  Problem p;
  int rc = validate_problem(a, &p);
  if (rc) return rc;
  if (p.B == 0 || p.n == 0) return SFA_OK;
  if (!q || !k || !v || !o) return fail(SFA_ERR_ARG, "sfa_fwd: NULL tensor");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(SFA_ERR_ARG, "sfa_fwd: tensors must be 16-byte aligned");
  SlotTable t;
  build_slots(a, &t, /*merge=*/true);
  ProfileScope ps("fwd_offsets", stream);
  return hip_status(launch_fwd_offsets(p, t, q, k, v, o, lse, stream), "sfa_fwd launch");
}

extern "C" int sfa_fwd_edges(const sfa_attn* a, const int32_t* edges, const int32_t* count, int width,
                             const void* q, const void* k, const void* v, void* o, float* lse,
                             void* stream) {
  clear_error();
  Problem p;
  if (!a) return fail(SFA_ERR_ARG, "problem is NULL");
  sfa_attn b = *a;
  b.window = 0;
  b.n_off = 0;
  int rc = validate_problem(&b, &p);
  if (rc) return rc;
  if (width < 1 || width > SFA_MAX_EDGE_WIDTH)
    return fail(SFA_ERR_ARG, "sfa_fwd_edges: width must be in [1, %d]", SFA_MAX_EDGE_WIDTH);
  if (p.B == 0 || p.n == 0) return SFA_OK;
  if (!q || !k || !v || !o || !edges || !count) return fail(SFA_ERR_ARG, "sfa_fwd_edges: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(edges) & 3u) || (reinterpret_cast<uintptr_t>(count) & 3u))
    return fail(SFA_ERR_ARG, "sfa_fwd_edges: misaligned pointer");
  ProfileScope ps("fwd_edges", stream);
  return hip_status(launch_fwd_edges(p, edges, count, width, q, k, v, o, lse, stream),
                    "sfa_fwd_edges launch");
}

// Edge-list problems ignore window and offsets, as sfa_fwd_edges does.
static int validate_edges_problem(const sfa_attn* a, Problem* p) {
  if (!a) return fail(SFA_ERR_ARG, "problem is NULL");
  sfa_attn b = *a;
  b.window = 0;
  b.n_off = 0;
  return validate_problem(&b, p);
}

extern "C" size_t sfa_bwd_edges_workspace_bytes(const sfa_attn* a, int width) {
  clear_error();
  Problem p;
  if (validate_edges_problem(a, &p)) return 0;
  if (width < 1 || width > SFA_MAX_EDGE_WIDTH) {
    fail(SFA_ERR_ARG, "sfa_bwd_edges_workspace_bytes: width must be in [1, %d]", SFA_MAX_EDGE_WIDTH);
    return 0;
  }
  return bwd_edges_workspace_layout(p, width, nullptr, nullptr, nullptr, nullptr, nullptr);
}

extern "C" int sfa_bwd_edges(const sfa_attn* a, const int32_t* edges, const int32_t* count, int width,
                             const int32_t* inv, const int32_t* inv_count, int inv_width, const void* q,
                             const void* k, const void* v, const float* lse, const void* dout, void* dq, void* dk,
                             void* dv, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  Problem p;
  int rc = validate_edges_problem(a, &p);
  if (rc) return rc;
  if (width < 1 || width > SFA_MAX_EDGE_WIDTH)
    return fail(SFA_ERR_ARG, "sfa_bwd_edges: width must be in [1, %d]", SFA_MAX_EDGE_WIDTH);
  if (inv_width < 1) return fail(SFA_ERR_ARG, "sfa_bwd_edges: inv_width must be >= 1");
  if (int64_t(p.n) * width > (int64_t(1) << 31) - 1)
    return fail(SFA_ERR_ARG, "sfa_bwd_edges: n * width exceeds int32 slot indices");
  if (p.B == 0 || p.n == 0) return SFA_OK;
  if (!q || !k || !v || !lse || !dout || !dq || !dk || !dv || !edges || !count || !inv || !inv_count)
    return fail(SFA_ERR_ARG, "sfa_bwd_edges: NULL pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(edges) & 3u) ||
      (reinterpret_cast<uintptr_t>(count) & 3u) || (reinterpret_cast<uintptr_t>(inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(inv_count) & 3u))
    return fail(SFA_ERR_ARG, "sfa_bwd_edges: misaligned pointer");
  const size_t need = bwd_edges_workspace_layout(p, width, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(SFA_ERR_CAPACITY, "sfa_bwd_edges: workspace needs %zu bytes (16-byte aligned), got %zu", need,
                ws_bytes);
  return hip_status(launch_bwd_edges(p, edges, count, width, inv, inv_count, inv_width, q, k, v, lse, dout, dq,
                                     dk, dv, workspace, stream),
                    "sfa_bwd_edges launch");
}

size_t sfa::bwd_workspace_bytes(const sfa_attn* a) {
  Problem p;
  if (validate_problem(a, &p)) return 0;
  SlotTable t;
  build_slots(a, &t);
  BwdWorkspace ws;
  return bwd_workspace_layout(p, t, nullptr, &ws);
}

extern "C" size_t sfa_bwd_workspace_bytes(const sfa_attn* a) {
  clear_error();
  return bwd_workspace_bytes(a);
}

namespace sfa {

int bwd_impl(const sfa_attn* a, const void* q, const void* k, const void* v, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* dd, const int32_t* base, double alpha, float* dtheta,
             void* workspace, size_t ws_bytes, void* stream, const char* fn) {
  Problem p;
  int rc = validate_problem(a, &p);
  if (rc) return rc;
  if (dtheta) {
    if (p.n_off > 0 && !base) return fail(SFA_ERR_ARG, "%s: dtheta needs the base rungs", fn);
    if (!std::isfinite(alpha)) return fail(SFA_ERR_ARG, "%s: alpha must be finite", fn);
  }
  SlotTable t;
  build_slots(a, &t);
  BwdWorkspace ws;
  const size_t need = bwd_workspace_layout(p, t, workspace, &ws);
  float base_f[SFA_MAX_OFFSETS];
  for (int i = 0; i < p.n_off; ++i) base_f[i] = base ? float(base[i]) : 0.f;
  if (p.B == 0 || p.n == 0) {
    // Nothing to sum: the reduce kernel over zero blocks writes zero dd/dtheta.
    if (!dd && !dtheta) return SFA_OK;
    ProfileScope ps("bwd_reduce", stream);
    return hip_status(launch_bwd_reduce(t, ws, base_f, alpha, dd, dtheta, stream), "bwd reduce launch");
  }
  if (!q || !k || !v || !lse || !dout || !dq || !dk || !dv) return fail(SFA_ERR_ARG, "%s: NULL tensor", fn);
  const void* ptrs[] = {q, k, v, lse, dout, dq, dk, dv};
  for (const void* x : ptrs)
    if (!aligned16(x)) return fail(SFA_ERR_ARG, "%s: tensors must be 16-byte aligned", fn);
  if (dd && (reinterpret_cast<uintptr_t>(dd) & 3u)) return fail(SFA_ERR_ARG, "%s: dd misaligned", fn);
  if (dtheta && (reinterpret_cast<uintptr_t>(dtheta) & 3u)) return fail(SFA_ERR_ARG, "%s: dtheta misaligned", fn);
  if (!workspace || ws_bytes < need || !aligned16(workspace))
    return fail(SFA_ERR_CAPACITY, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn, need, ws_bytes);
  {
    ProfileScope ps("bwd_query", stream);
    rc = hip_status(launch_bwd_query(p, t, q, k, v, lse, dout, dq, ws, dd || dtheta, stream), "bwd query launch");
    if (rc) return rc;
  }
  {
    ProfileScope ps("bwd_key", stream);
    rc = hip_status(launch_bwd_key(p, t, q, k, v, dout, dk, dv, ws, base_f, alpha, dd, dtheta, stream),
                    "bwd key launch");
    if (rc) return rc;
  }
  if ((dd || dtheta) && !bwd_key_reduces(p, t, true)) {
    ProfileScope ps("bwd_reduce", stream);
    rc = hip_status(launch_bwd_reduce(t, ws, base_f, alpha, dd, dtheta, stream), "bwd reduce launch");
  }
  return rc;
}

}  // namespace sfa

extern "C" int sfa_bwd(const sfa_attn* a, const void* q, const void* k, const void* v,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dd,
                       const int32_t* base, double alpha, float* dtheta, void* workspace,
                       size_t ws_bytes, void* stream) {
  clear_error();
  return bwd_impl(a, q, k, v, lse, dout, dq, dk, dv, dd, base, alpha, dtheta, workspace, ws_bytes, stream,
                  "sfa_bwd");
}
