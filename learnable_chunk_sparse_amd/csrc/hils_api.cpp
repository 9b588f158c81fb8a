// C ABI of the HiLS library: validation, workspace carving and the launch
// sequence of each operation. No device memory is allocated here; every
// launch goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/hils.h"
#include "hils_internal.h"

using hils::Dims;

namespace {

constexpr size_t ALIGN = 256;
inline size_t up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += up(bytes);
    return p;
  }
};

bool pow2ish_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// Structural checks shared by every op. Returns HILS_OK or the error.
hils_status check_problem(const hils_problem* p, int op) {
  if (p == nullptr) return HILS_ERR_INVALID;
  if (p->dtype != HILS_FP32 && p->dtype != HILS_BF16) return HILS_ERR_UNSUPPORTED;
  if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->d <= 0 || p->Nq <= 0 || p->Nk <= 0 ||
      p->S <= 0 || p->K <= 0 || p->W <= 0)
    return HILS_ERR_INVALID;
  if (p->Hq % p->Hkv != 0) return HILS_ERR_INVALID;
  if (p->r < 0 || (p->r > 0 && p->D <= 0)) return HILS_ERR_INVALID;
  if (!(p->scale >= 0.f) || std::isinf(p->scale)) return HILS_ERR_INVALID;
  if (op == HILS_OP_DECODE) {
    if (p->Nq != 1) return HILS_ERR_INVALID;
  } else {
    if (p->Nq != p->Nk) return HILS_ERR_INVALID;
  }
  if (p->d != 64 && p->d != 128) return HILS_ERR_UNSUPPORTED;
  if (p->S != 64) return HILS_ERR_UNSUPPORTED;
  if (p->qcal_shared != 0 && p->qcal_shared != 1) return HILS_ERR_INVALID;
  if (p->fwd_strategy < HILS_FWD_AUTO || p->fwd_strategy > HILS_FWD_CHUNK_MAJOR) return HILS_ERR_INVALID;
  const int G = p->Hq / p->Hkv;
  if (!pow2ish_group(G)) return HILS_ERR_UNSUPPORTED;
  if (p->r > 0) {
    if (!(p->r == 16 || p->r == 32 || p->r == 64)) return HILS_ERR_UNSUPPORTED;
    if (p->D % 32 != 0) return HILS_ERR_UNSUPPORTED;
  }
  if (op != HILS_OP_DECODE) {
    if (G > 4) return HILS_ERR_UNSUPPORTED;
    if (p->K > 32) return HILS_ERR_UNSUPPORTED;
  } else {
    if (p->K > 64) return HILS_ERR_UNSUPPORTED;
  }
  if ((long long)p->Nk > (1LL << 26)) return HILS_ERR_UNSUPPORTED;
  return HILS_OK;
}

// Checks of the landmark summary ops, which read only dtype, B, Hkv, d, Nk,
// S and scale.
hils_status check_landmark(const hils_problem* p) {
  if (p == nullptr) return HILS_ERR_INVALID;
  if (p->dtype != HILS_FP32 && p->dtype != HILS_BF16) return HILS_ERR_UNSUPPORTED;
  if (p->B <= 0 || p->Hkv <= 0 || p->d <= 0 || p->Nk <= 0 || p->S <= 0) return HILS_ERR_INVALID;
  if (!(p->scale >= 0.f) || std::isinf(p->scale)) return HILS_ERR_INVALID;
  if (p->d != 64 && p->d != 128) return HILS_ERR_UNSUPPORTED;
  if (p->S != 64) return HILS_ERR_UNSUPPORTED;
  if ((long long)p->Nk > (1LL << 26)) return HILS_ERR_UNSUPPORTED;
  return HILS_OK;
}

// chunk tensors (kL, e and their gradients) may be NULL when the sequence
// holds no complete chunk: they are empty and never touched
inline bool chunks_ok(const hils_problem* p, const void* a, const void* b) {
  return (p->Nk / p->S) == 0 || (a != nullptr && b != nullptr);
}

// 16-byte alignment of every non-null pointer (kernels that read or write
// rows as 16-byte vectors)
inline bool al16() { return true; }
template <typename... R>
inline bool al16(const void* a, R... rest) {
  return (reinterpret_cast<uintptr_t>(a) & 15) == 0 && al16(rest...);
}

// Without a complete chunk the kernels still form (and discard, or weight by
// zero) the landmark row and bias of chunk 0 for empty slots: a NULL kL / e
// is replaced by another input of the same dtype with at least d finite
// elements, which keeps those reads in bounds.
inline const void* or_stand_in(const void* x, const void* stand_in) { return x ? x : stand_in; }

Dims landmark_dims(const hils_problem* p) {
  Dims d{};
  d.dtype = p->dtype;
  d.B = p->B;
  d.Hkv = p->Hkv;
  d.d = p->d;
  d.N = p->Nk;
  d.S = p->S;
  d.C = p->Nk / p->S;
  d.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
  return d;
}

Dims dims_of(const hils_problem* p) {
  Dims d;
  d.dtype = p->dtype;
  d.B = p->B;
  d.Hq = p->Hq;
  d.Hkv = p->Hkv;
  d.G = p->Hq / p->Hkv;
  d.d = p->d;
  d.N = p->Nk;
  d.S = p->S;
  d.K = p->K;
  d.W = p->W;
  d.C = p->Nk / p->S;
  d.D = p->D;
  d.r = p->r;
  d.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->d);
  d.fwd_strategy = p->fwd_strategy;
  return d;
}

// Workspace layout of each op (the same function computes sizes and carves).
// Routing scratch with Q-Cal: the fp32 calibrated queries, or on the u path
// (hils::route_u_ok) u = W_down h in the same region (r <= d) and the
// W_up^T kL planes.
struct RouteWs {
  float* qhat = nullptr;  // q_hat [B, Hq, N, d], or u [B N, Hq r] on the u path
  uint16_t *klh = nullptr, *kll = nullptr;
};
void carve_route_ws(const Dims& d, Carver& c, RouteWs* out) {
  const size_t rows = (size_t)d.B * d.Hq * d.N;
  out->qhat = d.r > 0 ? (float*)c.take(rows * d.d * sizeof(float)) : nullptr;
  const size_t kp = hils::route_u_ok(d) ? (size_t)d.B * d.Hq * d.C * d.r * sizeof(uint16_t) : 0;
  out->klh = (uint16_t*)c.take(kp);
  out->kll = (uint16_t*)c.take(kp);
}
struct FwdWs {
  RouteWs rt;
  float* s_T;
  float* sel_lse;
  void* vt;
  // chunk-major strategy: the inverse index of the selection and the
  // per-(position, slot, head) chunk outputs
  hils::InvIndex ix;
  hils::CmItems items;
  void* part = nullptr;
};
size_t carve_fwd(const Dims& d, void* ws, FwdWs* out) {
  Carver c(ws);
  const size_t rows = (size_t)d.B * d.Hq * d.N;
  carve_route_ws(d, c, &out->rt);
  out->s_T = (float*)c.take(rows * d.K * sizeof(float));
  out->sel_lse = (float*)c.take(rows * sizeof(float));
  out->vt = c.take(hils::attn_fwd_vt_bytes(d));
  if (hils::fwd_strategy_of(d) == HILS_FWD_CHUNK_MAJOR) {
    const size_t ib = hils::inv_index_carve(d, nullptr, &out->ix, true);
    void* ibase = c.take(ib);
    hils::inv_index_carve(d, ibase, &out->ix, true);
    void* itb = c.take(hils::fwd_cm_items_carve(d, nullptr, &out->items));
    hils::fwd_cm_items_carve(d, itb, &out->items);
    out->part = c.take(hils::fwd_cm_part_bytes(d));
  }
  return c.used;
}
size_t carve_route(const Dims& d, void* ws, RouteWs* rt) {
  Carver c(ws);
  carve_route_ws(d, c, rt);
  return c.used;
}

// One Q-Cal pair shared by all heads (qcal_shared = 1): the per-head kernels
// read a copy of the pair per head, and the backward's per-head weight
// gradients are summed over the heads into the caller's [r, D] / [d, r]. The
// copies and those gradients live in a tail of the workspace, after the op's
// own scratch.
struct SharedQcal {
  void* wd = nullptr;    // [Hq, r, D] in the problem dtype
  void* wu = nullptr;    // [Hq, d, r]
  float* dwd = nullptr;  // [Hq, r, D] fp32 (backward)
  float* dwu = nullptr;  // [Hq, d, r] fp32 (backward)
};
size_t shared_tail(const hils_problem* p, const Dims& d, bool bwd, void* tail, SharedQcal* out) {
  if (p->qcal_shared != 1 || d.r == 0) return 0;
  Carver c(tail);
  const size_t es = d.dtype == HILS_BF16 ? 2 : 4;
  const size_t nd = (size_t)d.r * d.D, nu = (size_t)d.d * d.r;
  out->wd = c.take(d.Hq * nd * es);
  out->wu = c.take(d.Hq * nu * es);
  if (bwd) {
    out->dwd = static_cast<float*>(c.take(d.Hq * nd * sizeof(float)));
    out->dwu = static_cast<float*>(c.take(d.Hq * nu * sizeof(float)));
  }
  return c.used;
}
// per-head copies of a shared pair; W_down / W_up then point at them
hils_status expand_shared(const Dims& d, const SharedQcal& sq, const void*& W_down,
                          const void*& W_up, hipStream_t st) {
  if (sq.wd == nullptr) return HILS_OK;
  const size_t es = d.dtype == HILS_BF16 ? 2 : 4;
  if (hils::launch_repeat_heads(W_down, sq.wd, (size_t)d.r * d.D * es, d.Hq, st) != hipSuccess ||
      hils::launch_repeat_heads(W_up, sq.wu, (size_t)d.d * d.r * es, d.Hq, st) != hipSuccess)
    return HILS_ERR_HIP;
  W_down = sq.wd;
  W_up = sq.wu;
  return HILS_OK;
}

hils_status ws_check(void* ws, size_t have, size_t need) {
  if (need > have) return HILS_ERR_WORKSPACE;
  if (need > 0 && (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & (ALIGN - 1)) != 0))
    return HILS_ERR_WORKSPACE;
  return HILS_OK;
}

hils_status hip_status(hipError_t e) { return e == hipSuccess ? HILS_OK : HILS_ERR_HIP; }

// The prefill envelope: the forward's strategy fits the hardware (LDS, index
// limits) and the backward can train the same problem, so that
// hils_attn_fwd and hils_attn_bwd accept exactly the same problems.
bool fwd_fits_lds(const Dims& d) {
  if (hils::bwd_workspace(d) == (size_t)-1) return false;
  if (hils::fwd_strategy_of(d) == HILS_FWD_CHUNK_MAJOR) return hils::fwd_cm_ok(d);
  return hils::attn_fwd_lds_bytes(d) <= 160 * 1024;
}

// ---------------------------------------------------------------- timing hook
// events of the caller's hils_timing (per call; NULL = none) around step's launches
template <typename F>
hipError_t timed(const hils_timing* tm, int step, hipStream_t st, F&& launch) {
  void* a = tm ? tm->start[step] : nullptr;
  void* b = tm ? tm->stop[step] : nullptr;
  if (a == nullptr || b == nullptr) return launch();
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(a), st);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  return hipEventRecord(static_cast<hipEvent_t>(b), st);
}

// Q-Cal and routing of a prefill call (timed as two steps)
hils_status route_with_qcal(const hils_timing* tm, const Dims& d, const RouteWs& w, const void* q, const void* h,
                            const void* W_down, const void* W_up, const void* kL, const void* e,
                            int32_t* topk_idx, float* topk_score, float* sel_lse, hipStream_t st) {
  hils_status s;
  if (d.r > 0 && hils::route_u_ok(d)) {
    if ((s = hip_status(timed(tm, HILS_STEP_QCAL, st, [&] { return hils::launch_qcal(d, d.N, q, h, W_down, W_up, nullptr, w.qhat, st); }))) != HILS_OK)
      return s;
    return hip_status(timed(tm, HILS_STEP_ROUTE, st, [&] {
      hipError_t e2 = hils::launch_route_klp(d, W_up, kL, w.klh, w.kll, st);
      if (e2 != hipSuccess) return e2;
      hils::RouteU ru;
      ru.u = w.qhat;
      ru.klh = w.klh;
      ru.kll = w.kll;
      return hils::launch_route(d, q, false, kL, e, topk_idx, topk_score, sel_lse, st, ru);
    }));
  }
  if (d.r > 0) {
    if ((s = hip_status(timed(tm, HILS_STEP_QCAL, st, [&] { return hils::launch_qcal(d, d.N, q, h, W_down, W_up, w.qhat, nullptr, st); }))) != HILS_OK)
      return s;
    return hip_status(timed(tm, HILS_STEP_ROUTE, st, [&] { return hils::launch_route(d, w.qhat, true, kL, e, topk_idx, topk_score, sel_lse, st); }));
  }
  return hip_status(timed(tm, HILS_STEP_ROUTE, st, [&] { return hils::launch_route(d, q, d.dtype == HILS_FP32, kL, e, topk_idx, topk_score, sel_lse, st); }));
}

// ---------------------------------------------------------------- no-alloc scratch
// The scratch of hils_decode_noalloc: one copy per GPU the library runs on,
// held until the process ends. Host code never uses this name as an address
// (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current and kept in g_scratch_addr.
static __device__ __align__(256) unsigned char scratch[HILS_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[MAX_DEVICES];  // written once per device, under the mutex

// device address of the current device's scratch (set up on its first use)
hils_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return HILS_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return HILS_ERR_HIP;
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return HILS_OK;
}

}  // namespace

extern "C" {

const char* hils_status_string(hils_status s) {
  switch (s) {
    case HILS_OK: return "ok";
    case HILS_ERR_INVALID: return "invalid argument";
    case HILS_ERR_UNSUPPORTED: return "unsupported problem";
    case HILS_ERR_WORKSPACE: return "workspace too small or misaligned";
    case HILS_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

int32_t hils_version(void) { return 100; }

hils_status hils_workspace_size(const hils_problem* p, int32_t op, size_t* bytes) {
  if (bytes == nullptr) return HILS_ERR_INVALID;
  if (op < HILS_OP_ROUTE || op > HILS_OP_DECODE) return HILS_ERR_INVALID;
  hils_status s = check_problem(p, op);
  if (s != HILS_OK) return s;
  const Dims d = dims_of(p);
  SharedQcal sq;
  switch (op) {
    case HILS_OP_ROUTE: {
      RouteWs rt;
      *bytes = up(carve_route(d, nullptr, &rt)) + shared_tail(p, d, false, nullptr, &sq);
      return HILS_OK;
    }
    case HILS_OP_FWD: {
      if (!fwd_fits_lds(d)) return HILS_ERR_UNSUPPORTED;
      FwdWs w;
      *bytes = up(carve_fwd(d, nullptr, &w)) + shared_tail(p, d, false, nullptr, &sq);
      return HILS_OK;
    }
    case HILS_OP_BWD: {
      const size_t b = hils::bwd_workspace(d);
      if (b == (size_t)-1) return HILS_ERR_UNSUPPORTED;
      *bytes = up(b) + shared_tail(p, d, true, nullptr, &sq);
      return HILS_OK;
    }
    case HILS_OP_DECODE: {
      const size_t b = hils::decode_workspace(d);
      if (b == (size_t)-1) return HILS_ERR_UNSUPPORTED;
      *bytes = up(b) + shared_tail(p, d, false, nullptr, &sq);
      return HILS_OK;
    }
  }
  return HILS_ERR_INVALID;
}

hils_status hils_fwd_strategy_of(const hils_problem* p, int32_t* strategy) {
  if (strategy == nullptr) return HILS_ERR_INVALID;
  hils_status s = check_problem(p, HILS_OP_FWD);
  if (s != HILS_OK) return s;
  const Dims d = dims_of(p);
  if (!fwd_fits_lds(d)) return HILS_ERR_UNSUPPORTED;
  *strategy = hils::fwd_strategy_of(d);
  return HILS_OK;
}

hils_status hils_route(const hils_problem* p, const void* q, const void* kL, const void* e,
                       const void* h, const void* W_down, const void* W_up, int32_t* topk_idx,
                       float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  hils_status s = check_problem(p, HILS_OP_ROUTE);
  if (s != HILS_OK) return s;
  if (!q || !chunks_ok(p, kL, e) || !topk_idx) return HILS_ERR_INVALID;
  if (p->r > 0 && (!h || !W_down || !W_up)) return HILS_ERR_INVALID;
  kL = or_stand_in(kL, q);
  e = or_stand_in(e, q);
  const Dims d = dims_of(p);
  RouteWs rt;
  SharedQcal sq;
  const size_t base = up(carve_route(d, nullptr, &rt));
  const size_t need = base + shared_tail(p, d, false, nullptr, &sq);
  if ((s = ws_check(ws, ws_bytes, need)) != HILS_OK) return s;
  if (!al16(W_down, W_up)) return HILS_ERR_INVALID;
  carve_route(d, ws, &rt);
  shared_tail(p, d, false, static_cast<char*>(ws) + base, &sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = expand_shared(d, sq, W_down, W_up, st)) != HILS_OK) return s;
  return route_with_qcal(p->timing, d, rt, q, h, W_down, W_up, kL, e, topk_idx, topk_score, nullptr, st);
}

hils_status hils_attn_fwd(const hils_problem* p, const void* q, const void* k, const void* v,
                          const void* kL, const void* e, const void* h, const void* W_down,
                          const void* W_up, void* o, float* lse, int32_t* topk_idx, void* ws,
                          size_t ws_bytes, void* stream) {
  hils_status s = check_problem(p, HILS_OP_FWD);
  if (s != HILS_OK) return s;
  if (!q || !k || !v || !chunks_ok(p, kL, e) || !o || !lse || !topk_idx) return HILS_ERR_INVALID;
  if (p->r > 0 && (!h || !W_down || !W_up)) return HILS_ERR_INVALID;
  kL = or_stand_in(kL, k);
  e = or_stand_in(e, k);
  const Dims d = dims_of(p);
  if (!fwd_fits_lds(d)) return HILS_ERR_UNSUPPORTED;
  FwdWs w;
  SharedQcal sq;
  const size_t base = up(carve_fwd(d, nullptr, &w));
  const size_t need = base + shared_tail(p, d, false, nullptr, &sq);
  if ((s = ws_check(ws, ws_bytes, need)) != HILS_OK) return s;
  if (!al16(W_down, W_up)) return HILS_ERR_INVALID;
  carve_fwd(d, ws, &w);
  shared_tail(p, d, false, static_cast<char*>(ws) + base, &sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = expand_shared(d, sq, W_down, W_up, st)) != HILS_OK) return s;
  s = route_with_qcal(p->timing, d, w.rt, q, h, W_down, W_up, kL, e, topk_idx, w.s_T, w.sel_lse, st);
  if (s != HILS_OK) return s;
  const int Np = (d.N + 63) / 64 * 64;
  if (hils::fwd_strategy_of(d) != HILS_FWD_CHUNK_MAJOR)
    return hip_status(timed(p->timing, HILS_STEP_ATTN_FWD, st, [&] {
      hipError_t e2 = timed(p->timing, HILS_STEP_PREP, st, [&] { return hils::launch_vt_perm(d, v, w.vt, st); });
      if (e2 != hipSuccess) return e2;
      return timed(p->timing, HILS_STEP_WINDOW, st, [&] {
        return hils::launch_attn_fwd(d, q, k, w.vt, topk_idx, w.s_T, w.sel_lse, o, lse, st);
      });
    }));
  // chunk-major: V^T copy, inverse index and work items; selected chunks;
  // then window + fusion
  return hip_status(timed(p->timing, HILS_STEP_ATTN_FWD, st, [&] {
    hipError_t e2 = timed(p->timing, HILS_STEP_PREP, st, [&] {
      hipError_t e3 = hils::launch_vt_perm(d, v, w.vt, st);
      if (e3 != hipSuccess) return e3;
      e3 = hils::launch_inv_index(d, topk_idx, w.ix, st);
      if (e3 != hipSuccess) return e3;
      return hils::launch_cm_items(d, w.ix, w.items, st);
    });
    if (e2 != hipSuccess) return e2;
    e2 = timed(p->timing, HILS_STEP_CHUNKS, st, [&] {
      return hils::launch_fwd_cm_chunks(d, q, k, w.vt, Np, w.ix, w.items, w.part, st);
    });
    if (e2 != hipSuccess) return e2;
    return timed(p->timing, HILS_STEP_WINDOW, st, [&] {
      return hils::launch_fwd_cm_window(d, q, k, w.vt, Np, topk_idx, w.s_T, w.sel_lse, w.ix.rank, w.part, o, lse, st);
    });
  }));
}

hils_status hils_attn_bwd(const hils_problem* p, const void* q, const void* k, const void* v,
                          const void* kL, const void* e, const void* h, const void* W_down,
                          const void* W_up, const void* o, const float* lse,
                          const int32_t* topk_idx, const void* dO, float* dq, float* dk, float* dv,
                          float* dkL, float* de, float* dW_down, float* dW_up, float* dh,
                          void* ws, size_t ws_bytes, void* stream) {
  hils_status s = check_problem(p, HILS_OP_BWD);
  if (s != HILS_OK) return s;
  if (!q || !k || !v || !chunks_ok(p, kL, e) || !lse || !topk_idx || !dO || !dq || !dk || !dv ||
      !chunks_ok(p, dkL, de))
    return HILS_ERR_INVALID;
  if (p->r > 0 && (!h || !W_down || !W_up || !dW_down || !dW_up)) return HILS_ERR_INVALID;
  kL = or_stand_in(kL, k);
  e = or_stand_in(e, k);
  const Dims d = dims_of(p);
  const size_t b0 = hils::bwd_workspace(d);
  if (b0 == (size_t)-1) return HILS_ERR_UNSUPPORTED;
  SharedQcal sq;
  const size_t base = up(b0);
  const size_t need = base + shared_tail(p, d, true, nullptr, &sq);
  if ((s = ws_check(ws, ws_bytes, need)) != HILS_OK) return s;
  if (!al16(W_down, W_up)) return HILS_ERR_INVALID;
  shared_tail(p, d, true, static_cast<char*>(ws) + base, &sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = expand_shared(d, sq, W_down, W_up, st)) != HILS_OK) return s;
  return hip_status(timed(p->timing, HILS_STEP_BWD, st, [&] {
    // a shared pair: per-head gradients into the tail, then summed over heads
    float* gd = sq.dwd ? sq.dwd : dW_down;
    float* gu = sq.dwu ? sq.dwu : dW_up;
    hipError_t e2 = hils::launch_bwd(d, q, k, v, kL, e, h, W_down, W_up, o, lse, topk_idx, dO, dq,
                                     dk, dv, dkL, de, gd, gu, dh, ws, st);
    if (e2 != hipSuccess || sq.dwd == nullptr) return e2;
    e2 = hils::launch_sum_heads(sq.dwd, dW_down, (size_t)d.r * d.D, d.Hq, st);
    if (e2 != hipSuccess) return e2;
    return hils::launch_sum_heads(sq.dwu, dW_up, (size_t)d.d * d.r, d.Hq, st);
  }));
}

hils_status hils_decode(const hils_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seq_len, const void* kL, const void* e,
                        const void* h, const void* W_down, const void* W_up, void* o, float* lse,
                        int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  hils_status s = check_problem(p, HILS_OP_DECODE);
  if (s != HILS_OK) return s;
  if (!q || !k_cache || !v_cache || !chunks_ok(p, kL, e) || !o || !lse) return HILS_ERR_INVALID;
  if (p->r > 0 && (!h || !W_down || !W_up)) return HILS_ERR_INVALID;
  kL = or_stand_in(kL, k_cache);
  e = or_stand_in(e, k_cache);
  const Dims d = dims_of(p);
  const size_t b0 = hils::decode_workspace(d);
  if (b0 == (size_t)-1) return HILS_ERR_UNSUPPORTED;
  SharedQcal sq;
  const size_t base = up(b0);
  const size_t need = base + shared_tail(p, d, false, nullptr, &sq);
  if ((s = ws_check(ws, ws_bytes, need)) != HILS_OK) return s;
  if (!al16(W_down, W_up)) return HILS_ERR_INVALID;
  shared_tail(p, d, false, static_cast<char*>(ws) + base, &sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = expand_shared(d, sq, W_down, W_up, st)) != HILS_OK) return s;
  // the decode workspace starts with the fp32 calibrated queries when Q-Cal is on
  const void* qs = q;
  bool qf32 = d.dtype == HILS_FP32;
  if (d.r > 0) {
    float* qhat = static_cast<float*>(ws);
    if ((s = hip_status(timed(p->timing, HILS_STEP_QCAL, st, [&] { return hils::launch_qcal(d, 1, q, h, W_down, W_up, qhat, nullptr, st); }))) != HILS_OK)
      return s;
    qs = qhat;
    qf32 = true;
  }
  return hip_status(timed(p->timing, HILS_STEP_DECODE, st, [&] {
    return hils::launch_decode(d, qs, qf32, q, k_cache, v_cache, seq_len, nullptr, 0, kL, e, o, lse, topk_idx,
                               ws, st);
  }));
}

hils_status hils_decode_noalloc(const hils_problem* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_len, const void* kL,
                                const void* e, const void* h, const void* W_down, const void* W_up,
                                void* o, float* lse, int32_t* topk_idx, void* stream) {
  size_t need = 0;
  hils_status s = hils_workspace_size(p, HILS_OP_DECODE, &need);
  if (s != HILS_OK) return s;
  if (need > (size_t)HILS_NOALLOC_SCRATCH_BYTES) return HILS_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != HILS_OK) return s;
  // the same kernels as hils_decode, on the device's static scratch (every
  // scratch buffer of the decode is written before it is read: nothing to clear)
  return hils_decode(p, q, k_cache, v_cache, seq_len, kL, e, h, W_down, W_up, o, lse, topk_idx, ws,
                     (size_t)HILS_NOALLOC_SCRATCH_BYTES, stream);
}

hils_status hils_decode_paged(const hils_problem* p, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_len, const void* kL_pages, const void* e_pages,
                              const void* h, const void* W_down, const void* W_up, void* o,
                              float* lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                              void* stream) {
  hils_status s = check_problem(p, HILS_OP_DECODE);
  if (s != HILS_OK) return s;
  if (!q || !k_pages || !v_pages || !page_table || !seq_len || !chunks_ok(p, kL_pages, e_pages) || !o ||
      !lse)
    return HILS_ERR_INVALID;
  if (p->r > 0 && (!h || !W_down || !W_up)) return HILS_ERR_INVALID;
  if (max_pages <= 0 || (long long)max_pages * p->S != p->Nk) return HILS_ERR_INVALID;
  const Dims d = dims_of(p);
  const size_t b0 = hils::decode_workspace(d);
  if (b0 == (size_t)-1) return HILS_ERR_UNSUPPORTED;
  SharedQcal sq;
  const size_t base = up(b0);
  const size_t need = base + shared_tail(p, d, false, nullptr, &sq);
  if ((s = ws_check(ws, ws_bytes, need)) != HILS_OK) return s;
  if (!al16(W_down, W_up)) return HILS_ERR_INVALID;
  shared_tail(p, d, false, static_cast<char*>(ws) + base, &sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((s = expand_shared(d, sq, W_down, W_up, st)) != HILS_OK) return s;
  const void* qs = q;
  bool qf32 = d.dtype == HILS_FP32;
  if (d.r > 0) {
    float* qhat = static_cast<float*>(ws);
    if ((s = hip_status(timed(p->timing, HILS_STEP_QCAL, st, [&] { return hils::launch_qcal(d, 1, q, h, W_down, W_up, qhat, nullptr, st); }))) != HILS_OK)
      return s;
    qs = qhat;
    qf32 = true;
  }
  return hip_status(timed(p->timing, HILS_STEP_DECODE, st, [&] {
    return hils::launch_decode(d, qs, qf32, q, k_pages, v_pages, seq_len, page_table, max_pages,
                               kL_pages, e_pages, o, lse, topk_idx, ws, st);
  }));
}

hils_status hils_landmark_fwd(const hils_problem* p, const void* qL, const void* k, void* kL,
                              void* e, float* kL32, float* e32, void* stream) {
  hils_status s = check_landmark(p);
  if (s != HILS_OK) return s;
  if (!k || !chunks_ok(p, qL, qL) || !chunks_ok(p, kL, e)) return HILS_ERR_INVALID;
  if (!al16(qL, k, kL, kL32)) return HILS_ERR_INVALID;
  const Dims d = landmark_dims(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(timed(p->timing, HILS_STEP_LANDMARK_FWD, st, [&] {
    return hils::launch_landmark_fwd(d, qL, k, kL, e, kL32, e32, st);
  }));
}

hils_status hils_landmark_bwd(const hils_problem* p, const void* qL, const void* k,
                              const float* dkL, const float* de, float* dqL, float* dk,
                              void* stream) {
  hils_status s = check_landmark(p);
  if (s != HILS_OK) return s;
  if (!k || !dk || !chunks_ok(p, qL, dqL) || !chunks_ok(p, dkL, de)) return HILS_ERR_INVALID;
  if (!al16(qL, k, dkL, dqL, dk)) return HILS_ERR_INVALID;
  const Dims d = landmark_dims(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(timed(p->timing, HILS_STEP_LANDMARK_BWD, st, [&] {
    return hils::launch_landmark_bwd(d, qL, k, dkL, de, dqL, dk, st);
  }));
}

hils_status hils_hope(const hils_hope_params* p, const void* x, void* y, const int32_t* pos,
                      void* stream) {
  if (!p) return HILS_ERR_INVALID;
  if (p->dtype != HILS_FP32 && p->dtype != HILS_BF16) return HILS_ERR_INVALID;
  if (p->B < 0 || p->H < 0 || p->N < 0 || p->d <= 0) return HILS_ERR_INVALID;
  if (!std::isfinite(p->base) || !(p->base > 1.f) || p->train_len < 0) return HILS_ERR_INVALID;
  if ((p->interleaved != 0 && p->interleaved != 1) || (p->inverse != 0 && p->inverse != 1))
    return HILS_ERR_INVALID;
  if (p->d != 64 && p->d != 128) return HILS_ERR_UNSUPPORTED;
  if (p->B == 0 || p->H == 0 || p->N == 0) return HILS_OK;
  if (!x || !y) return HILS_ERR_INVALID;
  if (!al16(x, y)) return HILS_ERR_INVALID;
  const long long units = (long long)p->B * p->N * (p->d / 2) / (p->dtype == HILS_BF16 ? 8 : 4);
  if (units > 0x7fffff00LL) return HILS_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(timed(p->timing, HILS_STEP_HOPE, st, [&] {
    return hils::launch_hope(p->dtype, p->B, p->H, p->N, p->d, x, y, pos, (double)p->base,
                             p->train_len, p->interleaved == 1, p->inverse == 1, st);
  }));
}

}  // extern "C"
