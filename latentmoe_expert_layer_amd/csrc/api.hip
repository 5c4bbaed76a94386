// C ABI of the LatentMoE layer: argument validation, workspace carve-up and
// kernel launches.  No device memory is allocated and no host<->device copy or
// stream synchronisation happens here: every length that only the device knows
// (per-expert row counts, tile counts) stays on the device (the AgentX
// InferenceX v3 write-up, SGLang/TRT-LLM engine fixes: per-step device-to-host
// length syncs create decode bubbles).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <utility>

#include "../../include/latent_moe.h"
#include "kernels.h"

using lmoe::Tile;

namespace lmoe {
hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kernel})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({dev, kernel});
  return e;
}
}  // namespace lmoe

struct latent_moe_plan {
  int64_t T;
  int32_t E, k;
  int ids_mode;
  const int32_t* ids;
  const float* w;
  const int32_t* sorted_row;
  const int32_t* row_pos;
  const int32_t* offsets;
  Tile* tiles_s;
  int32_t* n_s;
  int64_t max_s;
  Tile* tiles_t;
  int32_t* n_t;
  int64_t max_t;
  int32_t* counts;  // per-chunk expert counts of the many-workgroup permutation
  hipEvent_t events[LMOE_N_STAGE_EVENTS];
  bool timing;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(LMOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Route workspace: [n_s][n_t] counters, then the two tile tables.
static_assert(LMOE_MAX_EXPERTS <= 4096, "the permutation kernels handle at most 4096 experts");

struct RouteLayout {
  size_t n_s, n_t, tiles_s, tiles_t, counts, total;
  int64_t max_s, max_t;
};

RouteLayout route_layout(int64_t T, int32_t E, int32_t k) {
  RouteLayout L{};
  const int64_t R = T * k;
  L.max_s = lmoe::max_tiles(R, E, lmoe::kSkinnyBM);
  L.max_t = lmoe::max_tiles(R, E, lmoe::kTiledBM);
  size_t off = 0;
  L.n_s = off;
  off = align_up(off + 4);
  L.n_t = off;
  off = align_up(off + 4);
  L.tiles_s = off;
  off = align_up(off + size_t(L.max_s) * sizeof(Tile));
  L.tiles_t = off;
  off = align_up(off + size_t(L.max_t) * sizeof(Tile));
  L.counts = off;  // per-chunk expert counts of the many-workgroup permutation
  off = align_up(off + size_t(lmoe::permute_scratch_ints(R, E)) * 4);
  L.total = off;
  return L;
}

// Forward workspace: bf16 intermediates z, hs, H, Y, rhat (and MXFP8 copies).
struct FwdLayout {
  size_t z, hs, H, Y, rhat, zq, zs, hq, hsc, total;
};

FwdLayout fwd_layout(int64_t T, int32_t k, int32_t l, int32_t I, int32_t S, int32_t Is, bool rows,
                     bool mx = false) {
  FwdLayout L{};
  const int64_t R = T * k;
  size_t off = 0;
  L.z = off;
  off = align_up(off + (rows ? 0 : size_t(T) * l * 2));
  L.hs = off;
  off = align_up(off + size_t(T) * S * Is * 2);
  L.H = off;  // bf16 H (MXFP4 experts: FC1 writes it only as MXFP8, below)
  off = align_up(off + (mx ? 0 : size_t(R) * I * 2));
  L.Y = off;
  off = align_up(off + size_t(R) * l * 2);
  L.rhat = off;
  off = align_up(off + (rows ? 0 : size_t(T) * l * 2));
  // MXFP8 copies of the expert-GEMM activations (MXFP4 weights only)
  L.zq = off;
  off = align_up(off + (mx ? size_t(T) * l : 0));
  L.zs = off;
  off = align_up(off + (mx ? size_t(T) * (l / 32) : 0));
  L.hq = off;
  off = align_up(off + (mx ? size_t(R) * I : 0));
  L.hsc = off;
  off = align_up(off + (mx ? size_t(R) * (I / 32) : 0));
  L.total = off;
  return L;
}

int check_route_dims(int64_t T, int32_t E, int32_t k, bool ids_mode) {
  if (T < 0) return fail(LMOE_EINVAL, "T=%lld < 0", (long long)T);
  if (k < 1 || k > LMOE_MAX_TOPK) return fail(LMOE_EINVAL, "k=%d outside [1,%d]", k, LMOE_MAX_TOPK);
  if (E < k) return fail(LMOE_EINVAL, "E=%d < k=%d", E, k);
  if (T * int64_t(k) >= (int64_t(1) << 31)) return fail(LMOE_EINVAL, "T*k=%lld >= 2^31", (long long)(T * k));
  if (!ids_mode && E > LMOE_MAX_EXPERTS_LOGITS)
    return fail(LMOE_EUNSUPPORTED, "E=%d > %d in logits mode", E, LMOE_MAX_EXPERTS_LOGITS);
  if (E > LMOE_MAX_EXPERTS || lmoe::permute_waves(E) == 0)
    return fail(LMOE_EUNSUPPORTED, "E=%d > %d", E, LMOE_MAX_EXPERTS);
  return LMOE_OK;
}

int check_fwd_dims(const latent_moe_plan* p, const lmoe_forward_args* a, bool rows) {
  if (a->l <= 0 || a->l % 64) return fail(LMOE_EINVAL, "l=%d is not a positive multiple of 64", a->l);
  if (a->I <= 0 || a->I % 64) return fail(LMOE_EINVAL, "I=%d is not a positive multiple of 64", a->I);
  if (a->l > 4096) return fail(LMOE_EUNSUPPORTED, "l=%d > 4096", a->l);
  if (a->S < 0 || a->S > LMOE_MAX_SHARED) return fail(LMOE_EINVAL, "S=%d outside [0,%d]", a->S, LMOE_MAX_SHARED);
  if (a->wfmt != LMOE_WFMT_BF16 && a->wfmt != LMOE_WFMT_MXFP4 && a->wfmt != LMOE_WFMT_MXFP4_W4A16)
    return fail(LMOE_EINVAL, "unknown wfmt %d", a->wfmt);
  if (a->wfmt != LMOE_WFMT_BF16) {
    if (a->l % 128 || a->I % 128)
      return fail(LMOE_EINVAL, "MXFP4 experts need l and I multiples of 128 (got %d, %d)", a->l, a->I);
    if (!a->s1 || !a->s3 || !a->s2) return fail(LMOE_EINVAL, "MXFP4 experts need scales s1, s3 and s2");
  }
  if (a->wlayout != LMOE_WLAYOUT_ROWS && a->wlayout != LMOE_WLAYOUT_TILED)
    return fail(LMOE_EINVAL, "unknown wlayout %d", a->wlayout);
  if (a->wlayout == LMOE_WLAYOUT_TILED &&
      (a->wfmt != LMOE_WFMT_BF16 || a->l % 128 || a->I % 128 || a->l < 256 || a->I < 256))
    return fail(LMOE_EUNSUPPORTED,
                "the tile-packed weight layout serves bf16 experts with l and I multiples of 128, >= 256 "
                "(got wfmt %d, l %d, I %d)", a->wfmt, a->l, a->I);
  if (rows) {
    if (a->w_out) return fail(LMOE_EINVAL, "rows mode (w_in == NULL) needs w_out == NULL");
    if (p->k != 1) return fail(LMOE_EINVAL, "rows mode needs k == 1 (got %d)", p->k);
    if (a->S != 0) return fail(LMOE_EINVAL, "rows mode has no shared experts (S=%d)", a->S);
  } else {
    if (!a->w_out) return fail(LMOE_EINVAL, "w_out is NULL but w_in is not");
    if (a->d <= 0 || a->d % 64) return fail(LMOE_EINVAL, "d=%d is not a positive multiple of 64", a->d);
    if (a->S > 0 && (a->Is <= 0 || a->Is % 64))
      return fail(LMOE_EINVAL, "Is=%d is not a positive multiple of 64", a->Is);
  }
  return LMOE_OK;
}


// ------------------------------------------------------------------ routing
// Checks the routing arguments; nothing is enqueued.  gate: the logits come
// from latent_moe_layer's router gate, so args->logits and ids_in are NULL.
int route_check(const lmoe_route_args* a, bool gate) {
  const bool ids_mode = !gate && a->ids_in != nullptr;
  int rc = check_route_dims(a->T, a->E, a->k, ids_mode);
  if (rc) return rc;
  if (a->T == 0) return LMOE_OK;  // empty batch: no pointer is read or checked
  if (gate) {
    if (a->logits || a->ids_in)
      return fail(LMOE_EINVAL, "latent_moe_layer computes the logits: route logits and ids_in must be NULL");
  } else if ((a->logits != nullptr) == ids_mode) {
    return fail(LMOE_EINVAL, "give exactly one of logits and ids_in");
  }
  if (ids_mode) {
    if (!a->weights_in) return fail(LMOE_EINVAL, "ids mode needs weights_in");
    if (a->k != 1) return fail(LMOE_EINVAL, "ids mode needs k == 1 (got %d)", a->k);
  } else if (!a->topk_ids || !a->topk_w) {
    return fail(LMOE_EINVAL, "logits mode needs topk_ids and topk_w");
  }
  if (!a->sorted_row || !a->row_pos || !a->offsets) return fail(LMOE_EINVAL, "NULL permutation output");
  const void* ptrs[] = {a->logits, a->ids_in, a->weights_in, a->topk_ids, a->topk_w,
                        a->sorted_row, a->row_pos, a->offsets, a->workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(LMOE_EINVAL, "device pointer %p is not 16-byte aligned", q);
  const size_t need = route_layout(a->T, a->E, a->k).total;
  if (!a->workspace || a->workspace_bytes < need)
    return fail(LMOE_EINVAL, "route workspace too small: %zu < %zu", a->workspace_bytes, need);
  return LMOE_OK;
}

// Fills the routing part of a plan from checked arguments (host only).
void fill_plan(latent_moe_plan* p, const lmoe_route_args* a, bool ids_mode) {
  p->T = a->T;
  p->E = a->E;
  p->k = a->k;
  p->ids_mode = ids_mode;
  if (a->T == 0) return;
  const RouteLayout L = route_layout(a->T, a->E, a->k);
  char* ws = static_cast<char*>(a->workspace);
  p->ids = ids_mode ? a->ids_in : a->topk_ids;
  p->w = ids_mode ? a->weights_in : a->topk_w;
  p->sorted_row = a->sorted_row;
  p->row_pos = a->row_pos;
  p->offsets = a->offsets;
  p->n_s = reinterpret_cast<int32_t*>(ws + L.n_s);
  p->n_t = reinterpret_cast<int32_t*>(ws + L.n_t);
  p->tiles_s = reinterpret_cast<Tile*>(ws + L.tiles_s);
  p->tiles_t = reinterpret_cast<Tile*>(ws + L.tiles_t);
  p->counts = reinterpret_cast<int32_t*>(ws + L.counts);
  p->max_s = L.max_s;
  p->max_t = L.max_t;
}

// Router top-k/softmax over `logits` (or the id copy in ids mode), then the
// permutation and the tile tables.  router_done: the top-k has already been
// enqueued (in the down-projection's launch); only the permutation is left.
int route_enqueue(const latent_moe_plan* p, const lmoe_route_args* a, const float* logits, hipStream_t s,
                  bool router_done = false) {
  const int64_t R = p->T * p->k;
  if (R == 0) return LMOE_OK;
  hipError_t e;
  if (router_done) {
  } else if (p->ids_mode) {
    if (a->topk_ids || a->topk_w) {
      e = lmoe::launch_copy_ids(a->ids_in, a->weights_in, R, a->topk_ids, a->topk_w, s);
      if (e != hipSuccess) return hip_fail(e, "copy_ids");
    }
  } else {
    e = lmoe::launch_router(logits, p->T, p->E, p->k, a->topk_ids, a->topk_w, s);
    if (e != hipSuccess) return hip_fail(e, "router");
  }
  e = lmoe::launch_permute(p->ids, R, p->E, a->offsets, a->sorted_row, a->row_pos, p->tiles_s, p->n_s,
                           p->tiles_t, p->n_t, p->counts, s);
  if (e != hipSuccess) return hip_fail(e, "permute");
  return LMOE_OK;
}

// ------------------------------------------------------------------ forward
// Checks the forward arguments against the plan; nothing is enqueued.
int fwd_check(const latent_moe_plan* p, const lmoe_forward_args* a) {
  const bool rows = a->w_in == nullptr;
  if (rows && !p->ids_mode) return fail(LMOE_EINVAL, "rows mode (w_in == NULL) needs an ids-mode plan");
  int rc = check_fwd_dims(p, a, rows);
  if (rc) return rc;
  if (p->T == 0) return LMOE_OK;  // empty batch: nothing is read, written or enqueued
  if (!a->x || !a->w1 || !a->w3 || !a->w2 || !a->y) return fail(LMOE_EINVAL, "NULL x, expert weight or y");
  if (a->S > 0 && (!a->ws1 || !a->ws3 || !a->ws2)) return fail(LMOE_EINVAL, "S > 0 needs ws1, ws3 and ws2");
  const void* ptrs[] = {a->x, a->w_in, a->w1, a->w3, a->w2, a->s1, a->s3, a->s2, a->norm_w,
                        a->w_out, a->ws1, a->ws3, a->ws2, a->y, a->workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(LMOE_EINVAL, "device pointer %p is not 16-byte aligned", q);
  if (a->wfmt == LMOE_WFMT_MXFP4_W4A16 && p->T * p->k > int64_t(32) * p->E && (a->l < 256 || a->I < 256))
    return fail(LMOE_EUNSUPPORTED,
                "MXFP4 w4a16 beyond T*k <= 32*E runs the tiled expert GEMMs: l and I >= 256 (got %d, %d)", a->l, a->I);
  const int32_t S = rows ? 0 : a->S;
  const size_t need = fwd_layout(p->T, p->k, a->l, a->I, S, S ? a->Is : 0, rows, a->wfmt == LMOE_WFMT_MXFP4).total;
  if (!a->workspace || a->workspace_bytes < need)
    return fail(LMOE_EINVAL, "forward workspace too small: %zu < %zu", a->workspace_bytes, need);
  return LMOE_OK;
}

struct FwdCtx {
  const latent_moe_plan* p;
  const lmoe_forward_args* a;
  hipStream_t s;
  bool rows, mx, w4a16, small;
  bool os;  // output-stationary experts: no permutation, H and Y in (token, slot) order
  int32_t S;
  FwdLayout L;
};

FwdCtx fwd_ctx(const latent_moe_plan* p, const lmoe_forward_args* a, hipStream_t s) {
  FwdCtx c{};
  c.p = p;
  c.a = a;
  c.s = s;
  c.rows = a->w_in == nullptr;
  c.mx = a->wfmt == LMOE_WFMT_MXFP4;
  c.w4a16 = a->wfmt == LMOE_WFMT_MXFP4_W4A16;
  c.small = p->T <= lmoe::kSmallM;
  c.S = c.rows ? 0 : a->S;
  c.L = fwd_layout(p->T, p->k, a->l, a->I, c.S, c.S ? a->Is : 0, c.rows, c.mx);
  return c;
}

// The latent down-projection z = x W_in^T as a dense GEMM over the forward
// workspace (MXFP4 w4a8 at large T: with z's MXFP8 copy from the epilogue,
// when the launch can write it).
lmoe::DenseGemm down_proj_gemm(const FwdCtx& c) {
  const lmoe_forward_args* a = c.a;
  char* ws = static_cast<char*>(a->workspace);
  lmoe::DenseGemm g{};
  g.M = int(c.p->T);
  g.N = int(a->l);
  g.nseg = 1;
  g.seg[0] = lmoe::GemmSeg{static_cast<const uint16_t*>(a->x), a->d, static_cast<const uint16_t*>(a->w_in), nullptr,
                           a->d, int(a->d)};
  g.gated = false;
  g.C = reinterpret_cast<uint16_t*>(ws + c.L.z);
  g.ldc = a->l;
  g.stream_c = true;
  if (c.mx && !c.small && lmoe::dense_gemm_quant_fits(g)) {
    g.Cq = reinterpret_cast<uint8_t*>(ws + c.L.zq);
    g.Cqs = reinterpret_cast<uint8_t*>(ws + c.L.zs);
  }
  return g;
}

// Stage 1 (and 2 at large T): the latent down-projection and the shared
// experts' gate/up on x.  route (small T only): the router's top-k of these
// logits runs in the same launch as the GEMMs.
int fwd_front(const FwdCtx& c, const lmoe_route_args* route = nullptr) {
  const latent_moe_plan* p = c.p;
  const lmoe_forward_args* a = c.a;
  const hipStream_t s = c.s;
  const FwdLayout& L = c.L;
  auto mark = [&](int i) -> hipError_t { return p->timing ? hipEventRecord(p->events[i], s) : hipSuccess; };
  char* ws = static_cast<char*>(a->workspace);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + L.z);
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + L.hs);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.H);
  uint16_t* Y = reinterpret_cast<uint16_t*>(ws + L.Y);
  uint16_t* rhat = reinterpret_cast<uint16_t*>(ws + L.rhat);
  const uint16_t* x = static_cast<const uint16_t*>(a->x);
  const int64_t T = p->T, R = p->T * p->k;
  const int64_t d = a->d, l = a->l, I = a->I, Is = a->Is;
  const int32_t S = c.S;
  const bool rows = c.rows, mx = c.mx, w4a16 = c.w4a16, small = c.small;
  (void)R, (void)H, (void)Y, (void)rhat, (void)hs, (void)z, (void)mx, (void)w4a16;
  hipError_t e;
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "event");
  // 1. latent down-projection, and the shared experts' gate/up on x
  if (!rows) {
    lmoe::DenseGemm g[2] = {};
    g[0] = down_proj_gemm(c);
    g[1].M = int(T);
    g[1].N = int(S * Is);
    g[1].nseg = 1;
    g[1].seg[0] = lmoe::GemmSeg{x, d, static_cast<const uint16_t*>(a->ws1), static_cast<const uint16_t*>(a->ws3),
                                d, int(d)};
    g[1].gated = true;
    g[1].C = hs;
    g[1].ldc = S * Is;
    g[1].stream_c = true;
    if (small && route) {
      // one launch for both GEMMs and the router's top-k, which does not
      // depend on them
      lmoe::FrontRoute fr{};
      fr.logits = route->logits;
      fr.T = T;
      fr.E = p->E;
      fr.k = p->k;
      fr.ids = route->topk_ids;
      fr.w = route->topk_w;
      e = lmoe::launch_small_dense_with_router(g, S > 0 ? 2 : 1, fr, s);
      if (e != hipSuccess) return hip_fail(e, "down-proj + router");
      if ((e = mark(1)) != hipSuccess) return hip_fail(e, "event");
    } else if (small) {
      // one launch for both: they read the same rows of x
      if ((e = lmoe::launch_small_dense(g, S > 0 ? 2 : 1, s)) != hipSuccess) return hip_fail(e, "down-proj");
      if ((e = mark(1)) != hipSuccess) return hip_fail(e, "event");
    } else {
      if ((e = lmoe::launch_dense_gemm(g[0], s)) != hipSuccess) return hip_fail(e, "down-proj");
      if ((e = mark(1)) != hipSuccess) return hip_fail(e, "event");
      if (S > 0 && (e = lmoe::launch_dense_gemm(g[1], s)) != hipSuccess) return hip_fail(e, "shared gate/up");
    }
  } else if ((e = mark(1)) != hipSuccess) {
    return hip_fail(e, "event");
  }
  return LMOE_OK;
}

// Stages 3-6: routed experts, combine (+ RMSNorm), up-projection.
int fwd_back(const FwdCtx& c) {
  const latent_moe_plan* p = c.p;
  const lmoe_forward_args* a = c.a;
  const hipStream_t s = c.s;
  const FwdLayout& L = c.L;
  auto mark = [&](int i) -> hipError_t { return p->timing ? hipEventRecord(p->events[i], s) : hipSuccess; };
  char* ws = static_cast<char*>(a->workspace);
  uint16_t* z = reinterpret_cast<uint16_t*>(ws + L.z);
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + L.hs);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.H);
  uint16_t* Y = reinterpret_cast<uint16_t*>(ws + L.Y);
  uint16_t* rhat = reinterpret_cast<uint16_t*>(ws + L.rhat);
  const uint16_t* x = static_cast<const uint16_t*>(a->x);
  const int64_t T = p->T, R = p->T * p->k;
  const int64_t d = a->d, l = a->l, I = a->I, Is = a->Is;
  const int32_t S = c.S;
  const bool rows = c.rows, mx = c.mx, w4a16 = c.w4a16, small = c.small;
  (void)R, (void)H, (void)Y, (void)rhat, (void)hs, (void)z, (void)mx, (void)w4a16;
  hipError_t e;
  // FC1's stage events are recorded by the launch itself, at the kernel's
  // start and end (the roofline figure of the grouped GEMM is that kernel's
  // own duration)
  hipEvent_t fc1_t0 = p->timing ? p->events[2] : nullptr, fc1_t1 = p->timing ? p->events[3] : nullptr;

  // 2-3. routed experts: grouped FC1 (gated) and FC2 over the permuted rows
  if (c.os) {
    // output-stationary: each workgroup finds its expert's rows by scanning
    // the router's ids; H and Y stay in (token, slot) order
    if (w4a16) {
      lmoe::W4Mlp m{};
      m.A = z;
      m.lda = l;
      m.a_row_div = p->k;
      m.W1 = static_cast<const uint8_t*>(a->w1);
      m.S1 = a->s1;
      m.W3 = static_cast<const uint8_t*>(a->w3);
      m.S3 = a->s3;
      m.W2 = static_cast<const uint8_t*>(a->w2);
      m.S2 = a->s2;
      m.Y = Y;
      m.ldy = l;
      m.os_ids = p->ids;
      m.os_R = R;
      if ((e = lmoe::launch_w4a16_mlp_os(m, p->E, s, fc1_t0, fc1_t1)) != hipSuccess)
        return hip_fail(e, "expert MLP (MXFP4 w4a16, output-stationary)");
    } else {
      lmoe::GroupedGemm f1{};
      f1.N = int(I);
      f1.K = int(l);
      f1.A = z;
      f1.lda = l;
      f1.a_row_div = p->k;
      f1.B = static_cast<const uint16_t*>(a->w1);
      f1.B3 = static_cast<const uint16_t*>(a->w3);
      f1.ldb = l;
      f1.b_estride = I * l;
      f1.gated = true;
      f1.C = H;
      f1.ldc = I;
      f1.os_ids = p->ids;
      f1.os_R = R;
      f1.packed = a->wlayout == LMOE_WLAYOUT_TILED;
      if ((e = lmoe::launch_grouped_skinny_os(f1, p->E, s, fc1_t0, fc1_t1)) != hipSuccess)
        return hip_fail(e, "expert FC1 (output-stationary)");
      lmoe::GroupedGemm f2 = f1;
      f2.N = int(l);
      f2.K = int(I);
      f2.A = H;
      f2.lda = I;
      f2.a_row_div = 1;
      f2.B = static_cast<const uint16_t*>(a->w2);
      f2.B3 = nullptr;
      f2.ldb = I;
      f2.b_estride = l * I;
      f2.gated = false;
      f2.C = Y;
      f2.ldc = l;
      if ((e = lmoe::launch_grouped_skinny_os(f2, p->E, s)) != hipSuccess)
        return hip_fail(e, "expert FC2 (output-stationary)");
    }
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  } else if (mx) {
    // w4a8: MXFP8 activations x MXFP4 weights on the block-scaled MFMA
    uint8_t* zq = reinterpret_cast<uint8_t*>(ws + L.zq);
    uint8_t* zs = reinterpret_cast<uint8_t*>(ws + L.zs);
    uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.hq);
    uint8_t* hsc = reinterpret_cast<uint8_t*>(ws + L.hsc);
    // (z's copy is written by the down-projection where it can)
    if ((rows || !down_proj_gemm(c).Cq) &&
        (e = lmoe::launch_quant_mxfp8(rows ? x : z, T, int(l), zq, zs, s)) != hipSuccess)
      return hip_fail(e, "quantise expert inputs");
    lmoe::GroupedMx m1{};
    m1.N = int(I);
    m1.K = int(l);
    m1.A = zq;
    m1.As = zs;
    m1.a_rows = p->sorted_row;
    m1.a_row_div = p->k;
    m1.B = static_cast<const uint8_t*>(a->w1);
    m1.Bs = a->s1;
    m1.B3 = static_cast<const uint8_t*>(a->w3);
    m1.B3s = a->s3;
    m1.gated = true;
    m1.C = nullptr;
    m1.ldc = I;
    m1.Cq = hq;    // FC1's epilogue writes H already quantised to MXFP8 (FC2's operand)
    m1.Cqs = hsc;
    m1.tiles = p->tiles_t;
    m1.ntiles = p->n_t;
    m1.max_tiles = p->max_t;
    m1.a_rows_n = T;
    if ((e = lmoe::launch_grouped_mx(m1, s, fc1_t0, fc1_t1)) != hipSuccess) return hip_fail(e, "expert FC1 (MXFP4)");
    lmoe::GroupedMx m2 = m1;
    m2.Cq = nullptr;
    m2.Cqs = nullptr;
    m2.N = int(l);
    m2.K = int(I);
    m2.A = hq;
    m2.As = hsc;
    m2.a_rows = nullptr;
    m2.a_row_div = 1;
    m2.B = static_cast<const uint8_t*>(a->w2);
    m2.Bs = a->s2;
    m2.B3 = nullptr;
    m2.B3s = nullptr;
    m2.gated = false;
    m2.C = Y;
    m2.ldc = l;
    m2.a_rows_n = R;
    if ((e = lmoe::launch_grouped_mx(m2, s)) != hipSuccess) return hip_fail(e, "expert FC2 (MXFP4)");
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  } else if (w4a16 && R > int64_t(32) * p->E) {
    // w4a16 beyond decode-shaped batches: the tiled grouped GEMMs, weights
    // upcast to bf16 on their way into LDS
    lmoe::GroupedGemm t1{};
    t1.N = int(I);
    t1.K = int(l);
    t1.A = rows ? x : z;
    t1.lda = l;
    t1.a_rows = p->sorted_row;
    t1.a_row_div = p->k;
    t1.B = static_cast<const uint16_t*>(a->w1);
    t1.B3 = static_cast<const uint16_t*>(a->w3);
    t1.w4 = true;
    t1.Bs = a->s1;
    t1.B3s = a->s3;
    t1.gated = true;
    t1.C = H;
    t1.ldc = I;
    t1.tiles = p->tiles_t;
    t1.ntiles = p->n_t;
    t1.max_tiles = p->max_t;
    t1.a_rows_n = T;
    if ((e = lmoe::launch_grouped_tiled(t1, s, fc1_t0, fc1_t1)) != hipSuccess)
      return hip_fail(e, "expert FC1 (MXFP4 w4a16, tiled)");
    lmoe::GroupedGemm t2 = t1;
    t2.N = int(l);
    t2.K = int(I);
    t2.A = H;
    t2.lda = I;
    t2.a_rows = nullptr;
    t2.a_row_div = 1;
    t2.B = static_cast<const uint16_t*>(a->w2);
    t2.B3 = nullptr;
    t2.Bs = a->s2;
    t2.B3s = nullptr;
    t2.gated = false;
    t2.C = Y;
    t2.ldc = l;
    t2.a_rows_n = R;
    if ((e = lmoe::launch_grouped_tiled(t2, s)) != hipSuccess) return hip_fail(e, "expert FC2 (MXFP4 w4a16, tiled)");
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  } else if (w4a16 && l == lmoe::kW4MlpWidth && I == lmoe::kW4MlpWidth) {
    // w4a16 at the 256 x 256 decode shape: FC1, SwiGLU and FC2 in one launch
    lmoe::W4Mlp m{};
    m.A = rows ? x : z;
    m.lda = l;
    m.a_rows = p->sorted_row;
    m.a_row_div = p->k;
    m.W1 = static_cast<const uint8_t*>(a->w1);
    m.S1 = a->s1;
    m.W3 = static_cast<const uint8_t*>(a->w3);
    m.S3 = a->s3;
    m.W2 = static_cast<const uint8_t*>(a->w2);
    m.S2 = a->s2;
    m.Y = Y;
    m.ldy = l;
    m.tiles = p->tiles_s;
    m.ntiles = p->n_s;
    m.max_tiles = p->max_s;
    if ((e = lmoe::launch_w4a16_mlp(m, s, fc1_t0, fc1_t1)) != hipSuccess)
      return hip_fail(e, "expert MLP (MXFP4 w4a16)");
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  } else if (w4a16) {
    // w4a16: bf16 activations, MXFP4 weights upcast in the weight-streaming kernel
    lmoe::GroupedW4 q1{};
    q1.N = int(I);
    q1.K = int(l);
    q1.A = rows ? x : z;
    q1.lda = l;
    q1.a_rows = p->sorted_row;
    q1.a_row_div = p->k;
    q1.B = static_cast<const uint8_t*>(a->w1);
    q1.Bs = a->s1;
    q1.B3 = static_cast<const uint8_t*>(a->w3);
    q1.B3s = a->s3;
    q1.gated = true;
    q1.C = H;
    q1.ldc = I;
    q1.tiles = p->tiles_s;
    q1.ntiles = p->n_s;
    q1.max_tiles = p->max_s;
    if ((e = lmoe::launch_grouped_w4a16(q1, s, fc1_t0, fc1_t1)) != hipSuccess)
      return hip_fail(e, "expert FC1 (MXFP4 w4a16)");
    lmoe::GroupedW4 q2 = q1;
    q2.N = int(l);
    q2.K = int(I);
    q2.A = H;
    q2.lda = I;
    q2.a_rows = nullptr;
    q2.a_row_div = 1;
    q2.B = static_cast<const uint8_t*>(a->w2);
    q2.Bs = a->s2;
    q2.B3 = nullptr;
    q2.B3s = nullptr;
    q2.gated = false;
    q2.C = Y;
    q2.ldc = l;
    if ((e = lmoe::launch_grouped_w4a16(q2, s)) != hipSuccess) return hip_fail(e, "expert FC2 (MXFP4 w4a16)");
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  } else {
    const bool skinny = R <= int64_t(32) * p->E;
    lmoe::GroupedGemm f1{};
    f1.N = int(I);
    f1.K = int(l);
    f1.A = rows ? x : z;
    f1.lda = l;
    f1.a_rows = p->sorted_row;
    f1.a_row_div = p->k;
    f1.B = static_cast<const uint16_t*>(a->w1);
    f1.B3 = static_cast<const uint16_t*>(a->w3);
    f1.ldb = l;
    f1.b_estride = I * l;
    f1.gated = true;
    f1.C = H;
    f1.ldc = I;
    f1.tiles = skinny ? p->tiles_s : p->tiles_t;
    f1.ntiles = skinny ? p->n_s : p->n_t;
    f1.max_tiles = skinny ? p->max_s : p->max_t;
    f1.packed = a->wlayout == LMOE_WLAYOUT_TILED;
    e = skinny ? lmoe::launch_grouped_skinny(f1, s, fc1_t0, fc1_t1) : lmoe::launch_grouped_tiled(f1, s, fc1_t0, fc1_t1);
    if (e != hipSuccess) return hip_fail(e, "expert FC1");

    lmoe::GroupedGemm f2 = f1;
    f2.N = int(l);
    f2.K = int(I);
    f2.A = H;
    f2.lda = I;
    f2.a_rows = nullptr;
    f2.a_row_div = 1;
    f2.B = static_cast<const uint16_t*>(a->w2);
    f2.B3 = nullptr;
    f2.ldb = I;
    f2.b_estride = l * I;
    f2.gated = false;
    f2.C = Y;
    f2.ldc = l;
    e = skinny ? lmoe::launch_grouped_skinny(f2, s) : lmoe::launch_grouped_tiled(f2, s);
    if (e != hipSuccess) return hip_fail(e, "expert FC2");
    if ((e = mark(4)) != hipSuccess) return hip_fail(e, "event");
  }

  // 4. weighted combine (+ RMSNorm); rows mode writes the weighted rows out
  if (rows) {
    e = lmoe::launch_combine(Y, p->row_pos, p->w, R, 1, int(l), nullptr, 0.0f, static_cast<uint16_t*>(a->y), s);
    if (e != hipSuccess) return hip_fail(e, "combine");
    for (int i = 5; i < LMOE_N_STAGE_EVENTS; ++i)
      if ((e = mark(i)) != hipSuccess) return hip_fail(e, "event");
    return LMOE_OK;
  }
  e = lmoe::launch_combine(Y, c.os ? nullptr : p->row_pos, p->w, T, p->k, int(l),
                           static_cast<const uint16_t*>(a->norm_w), a->norm_eps, rhat, s);
  if (e != hipSuccess) return hip_fail(e, "combine");
  if ((e = mark(5)) != hipSuccess) return hip_fail(e, "event");

  // 5. latent up-projection, K-concatenated with the shared experts' down-proj
  lmoe::DenseGemm u{};
  u.M = int(T);
  u.N = int(d);
  u.nseg = 1 + S;
  u.seg[0] = lmoe::GemmSeg{rhat, l, static_cast<const uint16_t*>(a->w_out), nullptr, l, int(l)};
  for (int i = 0; i < S; ++i)
    u.seg[1 + i] = lmoe::GemmSeg{hs + i * Is, S * Is, static_cast<const uint16_t*>(a->ws2) + i * d * Is, nullptr,
                                 Is, int(Is)};
  u.gated = false;
  u.C = static_cast<uint16_t*>(a->y);
  u.ldc = d;
  u.stream_c = true;
  e = small ? lmoe::launch_small_dense(&u, 1, s) : lmoe::launch_dense_gemm(u, s);
  if (e != hipSuccess) return hip_fail(e, "up-proj");
  if ((e = mark(6)) != hipSuccess) return hip_fail(e, "event");
  return LMOE_OK;
}


}  // namespace

extern "C" {

const char* latent_moe_last_error(void) { return g_err.c_str(); }

size_t latent_moe_route_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || k < 1 || E < k || E > LMOE_MAX_EXPERTS) return 0;
  return route_layout(T, E, k).total;
}

size_t latent_moe_forward_workspace_size(int64_t T, int32_t E, int32_t k, int32_t d, int32_t l, int32_t I,
                                         int32_t S, int32_t Is, int32_t wfmt, int32_t rows_mode) {
  (void)E;
  (void)d;
  if (T < 0 || k < 1 || l <= 0 || I <= 0 || S < 0 || (S > 0 && Is <= 0)) return 0;
  if (wfmt != LMOE_WFMT_BF16 && wfmt != LMOE_WFMT_MXFP4 && wfmt != LMOE_WFMT_MXFP4_W4A16) return 0;
  return fwd_layout(T, k, l, I, S, rows_mode ? 0 : Is, rows_mode != 0, wfmt == LMOE_WFMT_MXFP4).total;
}

int latent_moe_forward_workspace_layout(int64_t T, int32_t E, int32_t k, int32_t d, int32_t l, int32_t I,
                                        int32_t S, int32_t Is, int32_t wfmt, int32_t rows_mode,
                                        lmoe_forward_layout* out) {
  if (!out) return fail(LMOE_EINVAL, "NULL out");
  if (latent_moe_forward_workspace_size(T, E, k, d, l, I, S, Is, wfmt, rows_mode) == 0)
    return fail(LMOE_EINVAL, "invalid forward dimensions");
  const bool rows = rows_mode != 0;
  const bool mx = wfmt == LMOE_WFMT_MXFP4;
  const int32_t Sx = rows ? 0 : S;
  const FwdLayout L = fwd_layout(T, k, l, I, Sx, Sx ? Is : 0, rows, mx);
  lmoe_forward_layout o{};
  o.z = L.z;
  o.hs = L.hs;
  o.H = L.H;
  o.Y = L.Y;
  o.rhat = L.rhat;
  o.zq = L.zq;
  o.zs = L.zs;
  o.hq = L.hq;
  o.hsc = L.hsc;
  o.total = L.total;
  uint32_t w = LMOE_WS_Y;
  if (!rows) w |= LMOE_WS_Z | LMOE_WS_RHAT;
  if (!rows && Sx > 0) w |= LMOE_WS_HS;
  const bool fused_w4 = wfmt == LMOE_WFMT_MXFP4_W4A16 && l == lmoe::kW4MlpWidth && I == lmoe::kW4MlpWidth;
  if (!mx && !fused_w4) w |= LMOE_WS_H;
  if (mx) w |= LMOE_WS_ZQ | LMOE_WS_HQ;
  o.written = w;
  *out = o;
  return LMOE_OK;
}

int latent_moe_pack_weights(const void* src, void* dst, int32_t E, int32_t N, int32_t K, void* hip_stream) {
  if (!src || !dst) return fail(LMOE_EINVAL, "NULL src or dst");
  if (E < 1 || N < 1 || K < 1 || N % lmoe::kPackRows || K % 64)
    return fail(LMOE_EINVAL, "pack: E=%d N=%d K=%d (N a multiple of %d, K of 64)", E, N, K, lmoe::kPackRows);
  if (!aligned16(src) || !aligned16(dst)) return fail(LMOE_EINVAL, "pack: pointers must be 16-byte aligned");
  const size_t bytes = size_t(E) * size_t(N) * size_t(K) * 2;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return fail(LMOE_EINVAL, "pack: src and dst overlap");
  const hipError_t e = lmoe::launch_pack_weights(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), E,
                                                 N, K, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "pack weights");
  return LMOE_OK;
}

int latent_moe_route(const lmoe_route_args* a, void* hip_stream, latent_moe_plan** out_plan) {
  if (!a || !out_plan) return fail(LMOE_EINVAL, "NULL args or out_plan");
  *out_plan = nullptr;
  int rc = route_check(a, false);
  if (rc) return rc;
  latent_moe_plan* p = new (std::nothrow) latent_moe_plan();
  if (!p) return fail(LMOE_EINVAL, "out of host memory");
  const bool ids_mode = a->ids_in != nullptr;
  fill_plan(p, a, ids_mode);
  if ((rc = route_enqueue(p, a, a->logits, static_cast<hipStream_t>(hip_stream))) != LMOE_OK) {
    delete p;
    return rc;
  }
  *out_plan = p;
  return LMOE_OK;
}

int latent_moe_forward(const latent_moe_plan* p, const lmoe_forward_args* a, void* hip_stream) {
  if (!p || !a) return fail(LMOE_EINVAL, "NULL plan or args");
  int rc = fwd_check(p, a);
  if (rc) return rc;
  if (p->T == 0) return LMOE_OK;
  const FwdCtx c = fwd_ctx(p, a, static_cast<hipStream_t>(hip_stream));
  if ((rc = fwd_front(c)) != LMOE_OK) return rc;
  return fwd_back(c);
}

}  // extern "C"

namespace {

// latent_moe_layer's checks (nothing enqueued on failure).
int layer_check(const lmoe_route_args* r, const void* w_router, const float* logits, const lmoe_forward_args* f) {
  if (!r || !f) return fail(LMOE_EINVAL, "NULL route args or forward args");
  // with a router gate the logits are computed here; without one the route
  // arguments give them (or the ids), as for latent_moe_route
  const bool gate = w_router != nullptr;
  int rc = route_check(r, gate);
  if (rc) return rc;
  if (!f->w_in) return fail(LMOE_EINVAL, "latent_moe_layer needs the projections (w_in != NULL)");
  latent_moe_plan q{};
  fill_plan(&q, r, !gate && r->ids_in != nullptr);
  if ((rc = fwd_check(&q, f)) != LMOE_OK) return rc;
  if (r->T > 0) {
    if (gate) {
      if (!logits) return fail(LMOE_EINVAL, "NULL logits (the gate's output)");
      if (!aligned16(w_router) || !aligned16(logits))
        return fail(LMOE_EINVAL, "w_router and logits must be 16-byte aligned");
    } else if (logits) {
      return fail(LMOE_EINVAL, "without w_router the route arguments give the logits: logits must be NULL");
    }
  }
  return LMOE_OK;
}

// Enqueues the whole layer with the (checked) arguments into the plan `p`,
// which has been filled from them.
int layer_enqueue(latent_moe_plan* p, const lmoe_route_args* r, const void* w_router, float* logits,
                  const lmoe_forward_args* f, hipStream_t s) {
  if (p->T == 0) return LMOE_OK;
  const bool gate = w_router != nullptr;
  const FwdCtx c = fwd_ctx(p, f, s);
  int rc;
  if (!gate) {
    // given logits: at small T the top-k runs in the down-projection's launch
    // (it reads neither x nor z), leaving only the permutation before the experts
    const bool fuse = !p->ids_mode && c.small;
    if ((rc = fwd_front(c, fuse ? r : nullptr)) != LMOE_OK) return rc;
    if ((rc = route_enqueue(p, r, r->logits, s, fuse)) != LMOE_OK) return rc;
    return fwd_back(c);
  }
  if ((rc = fwd_front(c)) != LMOE_OK) return rc;
  // the router gate on the latent z (in the forward workspace): fp32 logits
  const uint16_t* z = reinterpret_cast<const uint16_t*>(static_cast<const char*>(f->workspace) + c.L.z);
  const uint16_t* wr = static_cast<const uint16_t*>(w_router);
  lmoe::DenseGemm g{};
  g.M = int(p->T);
  g.N = p->E;
  g.nseg = 1;
  g.seg[0] = lmoe::GemmSeg{z, f->l, wr, nullptr, f->l, f->l};
  g.gated = false;
  g.Cf = logits;
  g.ldc = p->E;
  const hipError_t e = c.small ? lmoe::launch_small_dense(&g, 1, s) : lmoe::launch_dense_gemm(g, s);
  if (e != hipSuccess) return hip_fail(e, "router gate");
  if ((rc = route_enqueue(p, r, logits, s)) != LMOE_OK) return rc;
  return fwd_back(c);
}

// ---------------------------------------------------- no-allocation variant
// Both workspaces of latent_moe_layer_noalloc live in this array.  Its name
// is a host-side stand-in: host code uses only the device address that
// hipGetSymbolAddress returns for the current device (one copy per GPU).
static __device__ __align__(256) unsigned char scratch[LMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on `dev` (looked up once per device,
// with that device current).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LMOE_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LMOE_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LMOE_OK;
}

}  // namespace

extern "C" {

int latent_moe_layer(const lmoe_route_args* r, const void* w_router, float* logits, const lmoe_forward_args* f,
                     void* hip_stream, latent_moe_plan** plan_io) {
  if (!plan_io) return fail(LMOE_EINVAL, "NULL plan_io");
  int rc = layer_check(r, w_router, logits, f);
  if (rc) return rc;
  latent_moe_plan q{};
  fill_plan(&q, r, w_router == nullptr && r->ids_in != nullptr);
  latent_moe_plan* p = *plan_io;
  const bool fresh = p == nullptr;
  if (fresh) {
    p = new (std::nothrow) latent_moe_plan();
    if (!p) return fail(LMOE_EINVAL, "out of host memory");
  } else {
    q.timing = p->timing;  // a reused plan keeps its stage events
    for (int i = 0; i < LMOE_N_STAGE_EVENTS; ++i) q.events[i] = p->events[i];
  }
  *p = q;
  *plan_io = p;
  rc = layer_enqueue(p, r, w_router, logits, f, static_cast<hipStream_t>(hip_stream));
  if (rc != LMOE_OK && fresh) {
    delete p;
    *plan_io = nullptr;
  }
  return rc;
}

int latent_moe_layer_os(const lmoe_route_args* r, const lmoe_forward_args* f, void* hip_stream) {
  if (!r || !f) return fail(LMOE_EINVAL, "NULL route args or forward args");
  if (!r->logits || r->ids_in) return fail(LMOE_EINVAL, "latent_moe_layer_os takes router logits (logits != NULL, ids_in == NULL)");
  int rc = check_route_dims(r->T, r->E, r->k, false);
  if (rc) return rc;
  if (!f->w_in) return fail(LMOE_EINVAL, "latent_moe_layer_os needs the projections (w_in != NULL)");
  latent_moe_plan q{};
  q.T = r->T;
  q.E = r->E;
  q.k = r->k;
  q.ids = r->topk_ids;
  q.w = r->topk_w;
  if ((rc = fwd_check(&q, f)) != LMOE_OK) return rc;
  if (r->T == 0) return LMOE_OK;
  if (r->T > lmoe::kSmallM)
    return fail(LMOE_EUNSUPPORTED, "latent_moe_layer_os serves decode-shaped batches (T=%lld > %d)",
                (long long)r->T, lmoe::kSmallM);
  if (r->T * r->k > lmoe::kOsMaxRows)
    return fail(LMOE_EUNSUPPORTED, "latent_moe_layer_os: T*k=%lld > %d", (long long)(r->T * r->k), lmoe::kOsMaxRows);
  if (f->wfmt == LMOE_WFMT_BF16) {
    if (f->l % 128 || f->I % 128)
      return fail(LMOE_EUNSUPPORTED, "latent_moe_layer_os with bf16 experts needs l and I multiples of 128");
  } else if (f->wfmt == LMOE_WFMT_MXFP4_W4A16) {
    if (f->l != lmoe::kW4MlpWidth || f->I != lmoe::kW4MlpWidth)
      return fail(LMOE_EUNSUPPORTED, "latent_moe_layer_os with MXFP4 w4a16 experts needs l = I = %d",
                  lmoe::kW4MlpWidth);
  } else {
    return fail(LMOE_EUNSUPPORTED, "latent_moe_layer_os runs bf16 or MXFP4 w4a16 experts");
  }
  if (!r->topk_ids || !r->topk_w) return fail(LMOE_EINVAL, "NULL topk_ids or topk_w");
  if (!aligned16(r->logits) || !aligned16(r->topk_ids) || !aligned16(r->topk_w))
    return fail(LMOE_EINVAL, "logits, topk_ids and topk_w must be 16-byte aligned");
  FwdCtx c = fwd_ctx(&q, f, static_cast<hipStream_t>(hip_stream));
  c.os = true;
  // the router's top-k runs in the down-projection's launch (small batches)
  if ((rc = fwd_front(c, r)) != LMOE_OK) return rc;
  return fwd_back(c);
}

int latent_moe_layer_noalloc(const lmoe_route_args* r, const void* w_router, float* logits,
                             const lmoe_forward_args* f, void* hip_stream) {
  if (!r || !f) return fail(LMOE_EINVAL, "NULL route args or forward args");
  if (r->workspace || r->workspace_bytes || f->workspace || f->workspace_bytes)
    return fail(LMOE_EINVAL, "latent_moe_layer_noalloc takes no workspaces (workspace must be NULL, size 0)");
  if (r->T < 0) return fail(LMOE_EINVAL, "T=%lld < 0", (long long)r->T);
  const bool gate = w_router != nullptr;
  const bool ids_mode = !gate && r->ids_in != nullptr;
  const size_t rws = latent_moe_route_workspace_size(r->T, r->E, r->k);
  const size_t fws = latent_moe_forward_workspace_size(r->T, r->E, r->k, f->d, f->l, f->I, f->S, f->Is, f->wfmt,
                                                       f->w_in == nullptr);
  if (r->T > 0 && (rws == 0 || fws == 0)) return fail(LMOE_EINVAL, "invalid dimensions");
  const size_t need = align_up(rws) + fws;
  if (need > size_t(LMOE_NOALLOC_SCRATCH_BYTES))
    return fail(LMOE_EUNSUPPORTED, "workspaces need %zu bytes, beyond the %zu-byte scratch of latent_moe_layer_noalloc",
                need, size_t(LMOE_NOALLOC_SCRATCH_BYTES));
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  int dev = 0;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  void* base = nullptr;
  int rc = scratch_on(dev, &base);
  if (rc) return rc;
  lmoe_route_args ra = *r;
  lmoe_forward_args fa = *f;
  ra.workspace = base;
  ra.workspace_bytes = align_up(rws);
  fa.workspace = static_cast<char*>(base) + align_up(rws);
  fa.workspace_bytes = fws;
  if ((rc = layer_check(&ra, w_router, logits, &fa)) != LMOE_OK) return rc;
  latent_moe_plan p{};  // on the stack: no host allocation, no stage events
  fill_plan(&p, &ra, ids_mode);
  return layer_enqueue(&p, &ra, w_router, logits, &fa, s);
}

void latent_moe_free(latent_moe_plan* p) { delete p; }

int latent_moe_plan_set_stage_events(latent_moe_plan* p, void* const* events, int n) {
  if (!p) return fail(LMOE_EINVAL, "NULL plan");
  if (!events || n == 0) {
    p->timing = false;
    return LMOE_OK;
  }
  if (n != LMOE_N_STAGE_EVENTS) return fail(LMOE_EINVAL, "need %d events, got %d", LMOE_N_STAGE_EVENTS, n);
  for (int i = 0; i < n; ++i) {
    if (!events[i]) return fail(LMOE_EINVAL, "event %d is NULL", i);
    p->events[i] = static_cast<hipEvent_t>(events[i]);
  }
  p->timing = true;
  return LMOE_OK;
}

}  // extern "C"
