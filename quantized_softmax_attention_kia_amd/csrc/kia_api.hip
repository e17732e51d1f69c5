// C ABI of libkia (declared in include/kia.h): argument checks, buffer layout,
// dispatch to the gfx950 kernels.
#include "kia.h"
#include "kia_launch.hpp"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

void set_err(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

constexpr size_t ALIGN = 256;
size_t round_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

kia_status_t check_params(const kia_params_t* p, kia::Problem* pr) {
  g_err[0] = '\0';
  if (!p) { set_err("params is NULL"); return KIA_ERR_INVALID_ARG; }
  if (p->B < 0 || p->H < 0 || p->T < 0) {
    set_err("B, H, T must be >= 0 (got %lld, %lld, %lld)", (long long)p->B, (long long)p->H, (long long)p->T);
    return KIA_ERR_INVALID_ARG;
  }
  if (p->D < 1) { set_err("D must be >= 1 (got %lld)", (long long)p->D); return KIA_ERR_INVALID_ARG; }
  if (p->D != 64 && p->D != 128) {
    set_err("head dim D=%lld is not built (supported: 64, 128)", (long long)p->D);
    return KIA_ERR_UNSUPPORTED;
  }
  if (p->K < 1 || p->K > 64) { set_err("K must be in 1..64 (got %d)", p->K); return KIA_ERR_INVALID_ARG; }
  if (p->causal != 0 && p->causal != 1) { set_err("causal must be 0 or 1"); return KIA_ERR_INVALID_ARG; }
  if (p->calib != KIA_CALIB_MINMAX && p->calib != KIA_CALIB_FWM) { set_err("bad calib %d", p->calib); return KIA_ERR_INVALID_ARG; }
  if (p->recon < KIA_RECON_LERP || p->recon > KIA_RECON_NEAREST_BINMEAN) { set_err("bad recon %d", p->recon); return KIA_ERR_INVALID_ARG; }
  if (p->ste != KIA_STE_WEIGHT && p->ste != KIA_STE_PROB) { set_err("bad ste %d", p->ste); return KIA_ERR_INVALID_ARG; }
  if (p->grad < KIA_GRAD_FULL || p->grad > KIA_GRAD_P1) { set_err("bad grad %d", p->grad); return KIA_ERR_INVALID_ARG; }
  if (p->dtype != KIA_F32 && p->dtype != KIA_BF16) { set_err("bad dtype %d", p->dtype); return KIA_ERR_INVALID_ARG; }
  if (!std::isfinite(p->scale) || p->scale < 0.f) { set_err("scale must be finite and >= 0"); return KIA_ERR_INVALID_ARG; }
  if (p->calib == KIA_CALIB_FWM && !(std::isfinite(p->tau) && p->tau > 0.f)) {
    set_err("FWM needs a finite tau > 0 (got %g)", (double)p->tau);
    return KIA_ERR_INVALID_ARG;
  }
  if (p->tail < KIA_TAIL_ZERO || p->tail > KIA_TAIL_RESOLVED) { set_err("bad tail %d", p->tail); return KIA_ERR_INVALID_ARG; }
  if (p->calib == KIA_CALIB_MINMAX && p->tail != KIA_TAIL_ZERO) {
    set_err("a tail policy other than zero needs FWM (MinMax has no window)");
    return KIA_ERR_INVALID_ARG;
  }
  const bool expb = p->recon >= KIA_RECON_SOFTMAX && p->recon <= KIA_RECON_EXP_FP8;
  if (expb && p->tail != KIA_TAIL_ZERO) {
    set_err("the exponential baselines have no window: tail must be zero");
    return KIA_ERR_INVALID_ARG;
  }
  const bool binmean = p->recon == KIA_RECON_BINMEAN || p->recon == KIA_RECON_NEAREST_BINMEAN;
  if (binmean && p->tail != KIA_TAIL_ZERO) {
    set_err("bin mean takes the zero tail only");
    return KIA_ERR_INVALID_ARG;
  }
  if (binmean && p->K > kia::BINM_MAXB - 1) {
    set_err("bin mean is built for K <= %d (got %d)", kia::BINM_MAXB - 1, p->K);
    return KIA_ERR_UNSUPPORTED;
  }
  // index ranges the kernels rely on: per-head offsets in int, grid size in int
  if (p->T > (1 << 20)) { set_err("T=%lld exceeds 2^20", (long long)p->T); return KIA_ERR_UNSUPPORTED; }
  const long long heads = (long long)p->B * (long long)p->H;
  if (p->B > 0 && heads / p->B != p->H) { set_err("B*H overflows"); return KIA_ERR_INVALID_ARG; }
  if (heads * ((p->T + 31) / 32) > 0x7fffffffLL) { set_err("grid too large"); return KIA_ERR_UNSUPPORTED; }
  pr->nheads = (int)heads;
  pr->T = (int)p->T;
  pr->D = (int)p->D;
  pr->K = p->K;
  pr->causal = p->causal;
  pr->tau = p->tau;
  pr->scale = p->scale > 0.f ? (double)p->scale : 1.0 / std::sqrt((double)p->D);
  pr->calib = expb ? kia::EXPB
              : p->calib == KIA_CALIB_MINMAX
                  ? kia::MINMAX
                  : (p->tail == KIA_TAIL_FLOOR ? kia::FWM_FLOOR : (p->tail == KIA_TAIL_RESOLVED ? kia::FWM_RES : kia::FWM));
  // resolved grid: table levels below the window down to b <= -104, where e^b rounds to 0 in
  // float, capped at LRES_MAX (keys below the table get their grid values computed)
  pr->lres = 0;
  pr->res_far = 0;
  if (pr->calib == kia::FWM_RES) {
    const double need = std::ceil((104.0 - (double)p->tau) * (double)p->K / (double)p->tau);
    pr->lres = need <= 0.0 ? 0 : (need >= (double)kia::LRES_MAX ? kia::LRES_MAX : (int)need);
    pr->res_far = need > (double)kia::LRES_MAX;
  }
  switch (p->recon) {
    case KIA_RECON_LERP: pr->mode = kia::LERP; break;
    case KIA_RECON_NEAREST: pr->mode = p->ste == KIA_STE_WEIGHT ? kia::NEAREST_W : kia::NEAREST_P; break;
    case KIA_RECON_SOFTMAX: pr->mode = kia::EXP32; break;
    case KIA_RECON_EXP_BF16: pr->mode = kia::EXPBF; break;
    case KIA_RECON_EXP_FP8: pr->mode = kia::EXPF8; break;
    case KIA_RECON_BINMEAN: pr->mode = kia::BINM; break;
    default: pr->mode = kia::NEARB; break;
  }
  pr->gk = p->grad == KIA_GRAD_DETACHED ? kia::GK_DETACHED : (p->grad == KIA_GRAD_P1 ? kia::GK_P1 : kia::GK_SUMS);
  pr->keepM = p->grad == KIA_GRAD_FULL || p->grad == KIA_GRAD_MAX_ONLY;
  pr->keepm = (p->grad == KIA_GRAD_FULL || p->grad == KIA_GRAD_MIN_ONLY) && pr->calib == kia::MINMAX;
  pr->bf16 = p->dtype == KIA_BF16;
  return KIA_OK;
}

struct Layout {
  size_t off[11];
  size_t rowrec_bytes;
  int nt;
  size_t tiles_per_head;
  size_t ws_off[4];
  size_t ws_bytes;
};

Layout layout(const kia::Problem& pr) {
  Layout L;
  const size_t N = (size_t)pr.nheads * pr.T;
  size_t o = 0;
  for (int i = 0; i < 9; ++i) { L.off[i] = o; o += round_up(N * 4); }
  L.off[9] = o;
  if (pr.mode == kia::NEAREST_P || pr.mode == kia::EXPBF) o += round_up(N * pr.D * 4);
  L.nt = (pr.T + 31) / 32;
  L.tiles_per_head = pr.causal ? (size_t)L.nt * (L.nt + 1) / 2 : (size_t)L.nt * L.nt;
  L.off[10] = o;
  o += (size_t)pr.nheads * L.tiles_per_head * 1024 * 4;
  L.rowrec_bytes = o;
  o = 0;
  const size_t tile_bytes = (size_t)pr.nheads * L.tiles_per_head * 1024 * 4;
  L.ws_off[0] = o;                       // key-major P tiles
  o += tile_bytes;
  L.ws_off[1] = o;                       // key-major dS tiles
  o += tile_bytes;
  L.ws_off[2] = o;                       // per-row mean of the detached dS (P1)
  o += round_up(N * 4);
  L.ws_off[3] = o;                       // per-row table of P values by index (coded P tiles)
  o += round_up(N * (size_t)(pr.K + 2) * 4);
  L.ws_bytes = o;
  return L;
}

kia::RowRec carve(const kia::Problem& pr, void* base) {
  const Layout L = layout(pr);
  char* b = static_cast<char*>(base);
  kia::RowRec r;
  r.M = reinterpret_cast<float*>(b + L.off[0]);
  r.m = reinterpret_cast<float*>(b + L.off[1]);
  r.amax = reinterpret_cast<int32_t*>(b + L.off[2]);
  r.amin = reinterpret_cast<int32_t*>(b + L.off[3]);
  r.nA = reinterpret_cast<int32_t*>(b + L.off[4]);
  r.nC = reinterpret_cast<int32_t*>(b + L.off[5]);
  r.WN = reinterpret_cast<float*>(b + L.off[6]);
  r.WL = reinterpret_cast<float*>(b + L.off[7]);
  r.E = reinterpret_cast<float*>(b + L.off[8]);
  r.OL = pr.mode == kia::NEAREST_P || pr.mode == kia::EXPBF ? reinterpret_cast<float*>(b + L.off[9]) : nullptr;
  r.S = reinterpret_cast<float*>(b + L.off[10]);
  r.nt = L.nt;
  r.tiles_per_head = L.tiles_per_head;
  return r;
}

kia_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return KIA_OK;
  set_err("%s: %s", what, hipGetErrorString(e));
  return KIA_ERR_HIP;
}

bool empty(const kia::Problem& pr) { return pr.nheads == 0 || pr.T == 0; }

}  // namespace

// The built-in workspace of kia_backward_noalloc.  Each GPU holds its own copy of this array
// (at its own address) from the library's load until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels are given the device address that
// hipGetSymbolAddress returns for the current device, taken once per device and kept below.
static __device__ __align__(256) unsigned char scratch[KIA_NOALLOC_WS_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[SCRATCH_MAX_DEVICES];

// The device address of the current device's copy of `scratch` (looked up on its first use).
kia_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "kia_backward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) {
    set_err("kia_backward_noalloc: device %d is beyond the %d this library keeps an address for", dev,
            SCRATCH_MAX_DEVICES);
    return KIA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "kia_backward_noalloc: hipGetSymbolAddress");
    if (!ptr) {
      set_err("kia_backward_noalloc: hipGetSymbolAddress gave a null address");
      return KIA_ERR_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return KIA_OK;
}

}  // namespace

extern "C" {

kia_status_t kia_workspace_size(const kia_params_t* p, size_t* rowrec_bytes, size_t* bwd_ws_bytes) {
  kia::Problem pr;
  kia_status_t st = check_params(p, &pr);
  if (st != KIA_OK) return st;
  const Layout L = layout(pr);
  if (rowrec_bytes) *rowrec_bytes = L.rowrec_bytes;
  if (bwd_ws_bytes) *bwd_ws_bytes = L.ws_bytes;
  return KIA_OK;
}

static kia_status_t forward_phase(const kia_params_t* p, const void* q, const void* k, const void* v, float* o,
                                  void* rowrec, void* stream, int phase, const char* name) {
  kia::Problem pr;
  kia_status_t st = check_params(p, &pr);
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  if (!q || !k || !v || (phase != 1 && !o) || !rowrec) { set_err("%s: null buffer", name); return KIA_ERR_INVALID_ARG; }
  kia::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.rec = carve(pr, rowrec);
  a.nheads = pr.nheads;
  a.T = pr.T; a.K = pr.K; a.causal = pr.causal; a.tau = pr.tau; a.scale = pr.scale; a.lres = pr.lres; a.res_far = pr.res_far;
  a.phase = phase;
  return hip_status(kia::launch_forward(pr, a, static_cast<hipStream_t>(stream)), name);
}

kia_status_t kia_forward(const kia_params_t* p, const void* q, const void* k, const void* v,
                         float* o, void* rowrec, void* stream) {
  return forward_phase(p, q, k, v, o, rowrec, stream, 0, "kia_forward");
}

kia_status_t kia_forward_scores(const kia_params_t* p, const void* q, const void* k, const void* v, void* rowrec,
                                void* stream) {
  return forward_phase(p, q, k, v, nullptr, rowrec, stream, 1, "kia_forward_scores");
}

kia_status_t kia_forward_weights(const kia_params_t* p, const void* q, const void* k, const void* v, float* o,
                                 void* rowrec, void* stream) {
  return forward_phase(p, q, k, v, o, rowrec, stream, 2, "kia_forward_weights");
}

static kia_status_t backward_stages(const kia_params_t* p, const void* q, const void* k, const void* v,
                                    const float* o, const void* d_o, const void* rowrec, float* dq, float* dk,
                                    float* dv, void* workspace, void* stream, int stages, const char* name) {
  kia::Problem pr;
  kia_status_t st = check_params(p, &pr);
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  const bool need_dq = stages & 1, need_kv = stages & 2;
  if (!q || !k || !v || !d_o || !rowrec || !workspace || (need_dq && (!o || !dq)) || (need_kv && (!dk || !dv))) {
    set_err("%s: null buffer", name);
    return KIA_ERR_INVALID_ARG;
  }
  const Layout L = layout(pr);
  kia::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dO = d_o;
  a.rec = carve(pr, const_cast<void*>(rowrec));
  a.dq = dq; a.dk = dk; a.dv = dv;
  char* ws = static_cast<char*>(workspace);
  a.pt = reinterpret_cast<float*>(ws + L.ws_off[0]);
  a.dst = reinterpret_cast<float*>(ws + L.ws_off[1]);
  a.rowmean = reinterpret_cast<float*>(ws + L.ws_off[2]);
  a.pcode = reinterpret_cast<uint8_t*>(ws + L.ws_off[0]);
  a.ptab = reinterpret_cast<float*>(ws + L.ws_off[3]);
  a.pc = kia::p_coded(pr.calib, pr.mode);
  a.nheads = pr.nheads;
  a.T = pr.T; a.K = pr.K; a.causal = pr.causal; a.tau = pr.tau; a.scale = (float)pr.scale; a.lres = pr.lres; a.res_far = pr.res_far;
  a.keepM = pr.keepM; a.keepm = pr.keepm; a.p1 = pr.gk == kia::GK_P1;
  return hip_status(kia::launch_backward(pr, a, static_cast<hipStream_t>(stream), stages), name);
}

kia_status_t kia_backward(const kia_params_t* p, const void* q, const void* k, const void* v,
                          const float* o, const void* d_o, const void* rowrec,
                          float* dq, float* dk, float* dv, void* workspace, void* stream) {
  return backward_stages(p, q, k, v, o, d_o, rowrec, dq, dk, dv, workspace, stream, 3, "kia_backward");
}

kia_status_t kia_backward_dq(const kia_params_t* p, const void* q, const void* k, const void* v,
                             const float* o, const void* d_o, const void* rowrec, float* dq,
                             void* workspace, void* stream) {
  return backward_stages(p, q, k, v, o, d_o, rowrec, dq, nullptr, nullptr, workspace, stream, 1, "kia_backward_dq");
}

kia_status_t kia_backward_dkdv(const kia_params_t* p, const void* q, const void* k, const void* v,
                               const void* d_o, const void* rowrec, float* dk, float* dv,
                               void* workspace, void* stream) {
  return backward_stages(p, q, k, v, nullptr, d_o, rowrec, nullptr, dk, dv, workspace, stream, 2,
                         "kia_backward_dkdv");
}

kia_status_t kia_backward_noalloc(const kia_params_t* p, const void* q, const void* k, const void* v,
                                  const float* o, const void* d_o, const void* rowrec, float* dq, float* dk,
                                  float* dv, void* stream) {
  kia::Problem pr;
  kia_status_t st = check_params(p, &pr);
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  const Layout L = layout(pr);
  if (L.ws_bytes > KIA_NOALLOC_WS_BYTES) {
    set_err("kia_backward_noalloc: these params need %zu bytes of workspace, above the built-in %zu "
            "(call kia_backward with a workspace)", L.ws_bytes, (size_t)KIA_NOALLOC_WS_BYTES);
    return KIA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != KIA_OK) return st;
  return backward_stages(p, q, k, v, o, d_o, rowrec, dq, dk, dv, ws, stream, 3, "kia_backward_noalloc");
}

static kia_status_t flash_params(const kia_params_t* p, kia::Problem* pr, const char* name) {
  kia_status_t st = check_params(p, pr);
  if (st != KIA_OK) return st;
  if (p->recon != KIA_RECON_SOFTMAX) {
    set_err("%s: the one-pass kernels compute exact softmax (recon %d given)", name, p->recon);
    return KIA_ERR_UNSUPPORTED;
  }
  return KIA_OK;
}

kia_status_t kia_flash_forward(const kia_params_t* p, const void* q, const void* k, const void* v, float* o,
                               float* rowstats, void* stream) {
  kia::Problem pr;
  kia_status_t st = flash_params(p, &pr, "kia_flash_forward");
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  if (!q || !k || !v || !o || !rowstats) { set_err("kia_flash_forward: null buffer"); return KIA_ERR_INVALID_ARG; }
  const size_t N = (size_t)pr.nheads * pr.T;
  kia::FlashArgs a{};
  a.nheads = pr.nheads;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.rowM = rowstats; a.rowW = rowstats + N; a.rowD = rowstats + 2 * N;
  a.T = pr.T; a.causal = pr.causal; a.scale = (float)pr.scale; a.scale_d = pr.scale;
  return hip_status(kia::launch_flash_forward(pr, a, static_cast<hipStream_t>(stream)), "kia_flash_forward launch");
}

kia_status_t kia_flash_backward(const kia_params_t* p, const void* q, const void* k, const void* v, const float* o,
                                const void* d_o, float* rowstats, float* dq, float* dk, float* dv, void* stream) {
  kia::Problem pr;
  kia_status_t st = flash_params(p, &pr, "kia_flash_backward");
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  if (!q || !k || !v || !o || !d_o || !rowstats || !dq || !dk || !dv) {
    set_err("kia_flash_backward: null buffer");
    return KIA_ERR_INVALID_ARG;
  }
  const size_t N = (size_t)pr.nheads * pr.T;
  kia::FlashArgs a{};
  a.nheads = pr.nheads;
  a.q = q; a.k = k; a.v = v; a.dO = d_o; a.o = const_cast<float*>(o);
  a.rowM = rowstats; a.rowW = rowstats + N; a.rowD = rowstats + 2 * N;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.T = pr.T; a.causal = pr.causal; a.scale = (float)pr.scale; a.scale_d = pr.scale;
  return hip_status(kia::launch_flash_backward(pr, a, static_cast<hipStream_t>(stream)), "kia_flash_backward launch");
}

kia_status_t kia_debug_bins(const kia_params_t* p, const void* rowrec, uint8_t* bins, void* stream) {
  kia::Problem pr;
  kia_status_t st = check_params(p, &pr);
  if (st != KIA_OK) return st;
  if (empty(pr)) return KIA_OK;
  if (!rowrec || !bins) { set_err("kia_debug_bins: null buffer"); return KIA_ERR_INVALID_ARG; }
  kia::BinsArgs a;
  a.rec = carve(pr, const_cast<void*>(rowrec));
  a.bins = bins;
  a.T = pr.T; a.K = pr.K; a.causal = pr.causal; a.tau = pr.tau;
  return hip_status(kia::launch_bins(pr, a, static_cast<hipStream_t>(stream)), "kia_debug_bins launch");
}

const char* kia_status_string(int s) {
  switch (s) {
    case KIA_OK: return "KIA_OK";
    case KIA_ERR_INVALID_ARG: return "KIA_ERR_INVALID_ARG";
    case KIA_ERR_UNSUPPORTED: return "KIA_ERR_UNSUPPORTED";
    case KIA_ERR_WORKSPACE: return "KIA_ERR_WORKSPACE";
    case KIA_ERR_HIP: return "KIA_ERR_HIP";
  }
  return "KIA_ERR_UNKNOWN";
}

const char* kia_last_error(void) { return g_err; }

}  // extern "C"
