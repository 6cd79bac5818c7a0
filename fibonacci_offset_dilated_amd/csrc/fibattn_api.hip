// C ABI of the Fibonacci-offset dilated sparse attention library: argument validation,
// the exact offset-table builder, the per-layer schedules and kernel dispatch.
//
// Rules implemented here ("Depth-Staggered Fibonacci Spacing for Sparse Attention",
// gist.science summaries of arXiv 2606.28560):
//   Method > Architecture and attention mechanism: d_k = alpha * f_k per base offset f_k;
//   Results 2 (efficiency): static schedules take integer offsets, learned ones interpolate;
//   Method > Experimental variables: Fixed (alpha = 1), Staggered-linear (0.5 at layer 0 to
//   1.5 at the last layer) and Staggered-coprime (the linear values reassigned by
//   l -> 7l mod L) schedules.
#include <mutex>
#include <math.h>
#include <string.h>

#include <type_traits>

#include "../../include/fibattn.h"
#include "fib_launch.h"

using namespace fib;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int64_t B, int64_t H, int64_t N, int64_t D, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FIB_ERR_SHAPE;
  if (D != kD) return FIB_ERR_HEAD_DIM;
  if (dtype != FIB_F32 && dtype != FIB_BF16) return FIB_ERR_DTYPE;
  if (N > 0x7fffffffLL) return FIB_ERR_SHAPE;
  if (B > (1LL << 31) || H > (1LL << 31) || B * H > (1LL << 31)) return FIB_ERR_SHAPE;
  const int64_t BH = B * H;
  if ((double)BH * (double)N * (double)D > 9.0e18) return FIB_ERR_SHAPE;
  // one block per 64 queries per head in the general kernels
  if ((double)BH * (double)((N + 63) / 64) > 2147483647.0) return FIB_ERR_SHAPE;
  return FIB_OK;
}

int check_base(const int32_t* base, int n_base) {
  if (base == nullptr) return FIB_ERR_NULL;
  if (n_base < 1 || n_base > FIB_MAX_BASE) return FIB_ERR_BASE;
  for (int e = 0; e < n_base; ++e) {
    if (base[e] < 1 || base[e] > (1 << 24)) return FIB_ERR_BASE;
    if (e > 0 && base[e] <= base[e - 1]) return FIB_ERR_BASE;
  }
  return FIB_OK;
}

int check_scalars(int W, float alpha, float theta, int mode) {
  if (W < 1) return FIB_ERR_WINDOW;
  if (!isfinite(alpha) || alpha <= 0.f) return FIB_ERR_ALPHA;
  if (!isfinite(theta) || theta <= 0.f) return FIB_ERR_THETA;
  if (mode != FIB_INT && mode != FIB_INTERP) return FIB_ERR_MODE;
  return FIB_OK;
}

Rope make_rope(float theta) {
  Rope r;
  for (int j = 0; j < kHalf; ++j)
    r.rev[j] = pow((double)theta, -2.0 * (double)j / (double)kD) / (2.0 * M_PI);
  return r;
}

// fp32 nearest to p / q (q > 0), ties to an even significand.
float f32_nearest_ratio(int64_t p, int64_t q) {
  const float g = (float)((double)p / (double)q);
  float best = g;
  double best_err = -1.0;
  const float cand[3] = {nextafterf(g, -INFINITY), g, nextafterf(g, INFINITY)};
  for (float c : cand) {
    const double err = fabs((double)c * (double)q - (double)p);  // exact: 24 + 31 bits
    bool better = best_err < 0.0 || err < best_err;
    if (!better && err == best_err) {
      uint32_t u;
      memcpy(&u, &c, 4);
      better = (u & 1u) == 0;
    }
    if (better) {
      best = c;
      best_err = err;
    }
  }
  return best;
}

// ---- fixed scratch of the no-alloc backward -------------------------------------------------
// The workspace of fib_sparse_attn_bwd_noalloc: a device array in this code object, loaded
// (and held until the process ends) on each GPU the library runs on. Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in for the symbol):
// it uses the device address that hipGetSymbolAddress returns, once per device, with that
// device current.
constexpr size_t kScratchBytes = FIB_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FIB_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FIB_ERR_LAUNCH;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return FIB_OK;
}

}  // namespace

extern "C" {

const char* fib_status_string(int status) {
  switch (status) {
    case FIB_OK: return "ok";
    case FIB_ERR_NULL: return "a required pointer is NULL";
    case FIB_ERR_SHAPE: return "bad shape (B, H, N must be >= 1 and within index range)";
    case FIB_ERR_HEAD_DIM: return "unsupported head size (D must be 64)";
    case FIB_ERR_DTYPE: return "bad dtype (FIB_F32 or FIB_BF16)";
    case FIB_ERR_WINDOW: return "window W must be >= 1";
    case FIB_ERR_ALPHA: return "alpha must be finite and > 0";
    case FIB_ERR_BASE: return "base must hold 1..32 strictly increasing offsets in [1, 2^24]";
    case FIB_ERR_THETA: return "rope_theta must be finite and > 0";
    case FIB_ERR_MODE: return "mode must be FIB_INT or FIB_INTERP";
    case FIB_ERR_ALIGN: return "device pointers must be 16-byte aligned";
    case FIB_ERR_WORKSPACE: return "backward workspace missing or too small";
    case FIB_ERR_LAUNCH: return "kernel launch failed";
    case FIB_ERR_SCHEDULE: return "bad schedule kind, layer or layer count";
    case FIB_ERR_CAPACITY: return "output array too small";
    case FIB_ERR_SCRATCH: return "backward workspace need exceeds the no-alloc scratch (64 MiB)";
    default: return "unknown status";
  }
}

int fib_schedule_alpha(int schedule, int layer, int n_layers, float* out_alpha) {
  if (out_alpha == nullptr) return FIB_ERR_NULL;
  if (n_layers < 1 || layer < 0 || layer >= n_layers) return FIB_ERR_SCHEDULE;
  switch (schedule) {
    case FIB_SCHED_FIXED:
      *out_alpha = 1.0f;
      return FIB_OK;
    case FIB_SCHED_LINEAR:
      if (n_layers < 2) return FIB_ERR_SCHEDULE;
      // 0.5 + l / (L - 1) = (L - 1 + 2 l) / (2 (L - 1))
      *out_alpha = f32_nearest_ratio((int64_t)(n_layers - 1) + 2 * (int64_t)layer, 2 * (int64_t)(n_layers - 1));
      return FIB_OK;
    case FIB_SCHED_COPRIME: {
      if (n_layers < 2 || n_layers % 7 == 0) return FIB_ERR_SCHEDULE;
      const int src = (int)((7LL * layer) % n_layers);
      *out_alpha = f32_nearest_ratio((int64_t)(n_layers - 1) + 2 * (int64_t)src, 2 * (int64_t)(n_layers - 1));
      return FIB_OK;
    }
    default:
      return FIB_ERR_SCHEDULE;
  }
}

int fib_sparse_attn_offset_table(float alpha, const int32_t* base, int n_base, int W, int mode,
                                 int32_t* out_dist, float* out_w, int32_t* out_f, int* out_n) {
  if (out_dist == nullptr || out_w == nullptr || out_f == nullptr || out_n == nullptr) return FIB_ERR_NULL;
  int st = check_base(base, n_base);
  if (st) return st;
  st = check_scalars(W, alpha, 1.f, mode);
  if (st) return st;
  Table t;
  build_table(alpha, base, n_base, W, mode, &t);
  for (int e = 0; e < t.n; ++e) {
    out_dist[e] = t.dist[e];
    out_w[e] = t.w[e];
    out_f[e] = (int32_t)t.f[e];
  }
  *out_n = t.n;
  return FIB_OK;
}

int fib_sparse_attn_index_set(int64_t N, int W, float alpha, const int32_t* base, int n_base, int mode,
                              int32_t* out, int64_t out_cols, void* stream) {
  if (out == nullptr) return FIB_ERR_NULL;
  if (N < 1 || N > 0x7fffffffLL) return FIB_ERR_SHAPE;
  int st = check_base(base, n_base);
  if (st) return st;
  st = check_scalars(W, alpha, 1.f, mode);
  if (st) return st;
  Table t;
  build_table(alpha, base, n_base, W, mode, &t);
  if (out_cols != (int64_t)W + t.n) return FIB_ERR_CAPACITY;
  if ((double)N * (double)out_cols > 4.0e18) return FIB_ERR_SHAPE;
  if (launch_index_set(out, N, W, t, out_cols, (hipStream_t)stream) != hipSuccess) return FIB_ERR_LAUNCH;
  return FIB_OK;
}

}  // extern "C"

namespace {

// Where alpha comes from: one host value; or device memory (one value per layer) together
// with the range the launch is planned for; or (calls over several layers) one host value
// per layer. The last two build their tables on the device into the caller's plan buffer
// (one DevPlan per layer).
struct AlphaArg {
  bool dev;
  float host;
  const float* ptr;        // device alphas [layers]
  const float* host_list;  // host alphas [layers]
  int64_t layers;
  float lo, hi;
  void* plan;
  size_t plan_bytes;
  bool uses_plan() const { return dev || host_list != nullptr; }
};

int check_alpha(const AlphaArg& al) {
  if (al.layers < 1 || al.layers > kMaxLayers) return FIB_ERR_SHAPE;
  if (!al.uses_plan()) return isfinite(al.host) && al.host > 0.f ? FIB_OK : FIB_ERR_ALPHA;
  if (al.plan == nullptr || (al.dev && al.ptr == nullptr)) return FIB_ERR_NULL;
  if (al.dev) {
    if (!isfinite(al.lo) || !isfinite(al.hi) || al.lo <= 0.f || al.hi < al.lo) return FIB_ERR_ALPHA;
    if ((uintptr_t)al.ptr & 3u) return FIB_ERR_ALIGN;
  } else {
    for (int64_t l = 0; l < al.layers; ++l)
      if (!isfinite(al.host_list[l]) || al.host_list[l] <= 0.f) return FIB_ERR_ALPHA;
  }
  if (!aligned16(al.plan)) return FIB_ERR_ALIGN;
  if (al.plan_bytes < (size_t)al.layers * sizeof(DevPlan)) return FIB_ERR_WORKSPACE;
  return FIB_OK;
}

// The largest alpha a (checked) call can use: the host value, the top of the declared range
// (device alphas are clamped into it) or the largest of the host list.
float alpha_max(const AlphaArg& al) {
  if (!al.uses_plan()) return al.host;
  if (al.dev) return al.hi;
  float m = al.host_list[0];
  for (int64_t l = 1; l < al.layers; ++l) m = fmaxf(m, al.host_list[l]);
  return m;
}

// The call's table: built on the host, or by a kernel (one thread per layer) enqueued on the
// stream ahead of the attention kernels, which then read it from the plan.
template <typename Args>
int set_table(Args& a, const AlphaArg& al, const int32_t* base, int n_base) {
  a.layers = (int)al.layers;
  a.heads_per_plan = (int)(a.BH / al.layers);
  if (!al.uses_plan()) {
    build_table(al.host, base, n_base, a.W, a.mode, &a.tab);
    return FIB_OK;
  }
  memset(&a.tab, 0, sizeof(a.tab));
  BaseList bl;
  memset(&bl, 0, sizeof(bl));
  for (int e = 0; e < n_base; ++e) bl.v[e] = base[e];
  AlphaList hl;
  memset(&hl, 0, sizeof(hl));
  float lo = al.lo, hi = al.hi;
  if (!al.dev) {
    // host values: the kernels are planned for exactly their range
    lo = hi = al.host_list[0];
    for (int64_t l = 0; l < al.layers; ++l) {
      hl.v[l] = al.host_list[l];
      lo = fminf(lo, hl.v[l]);
      hi = fmaxf(hi, hl.v[l]);
    }
  }
  if (launch_dev_plan((DevPlan*)al.plan, al.dev ? al.ptr : nullptr, hl, (int)al.layers, lo, hi, bl, n_base, a.W,
                      a.mode, a.N, a.stream) != hipSuccess)
    return FIB_ERR_LAUNCH;
  a.plan = (const DevPlan*)al.plan;
  a.alpha_lo = lo;
  a.alpha_hi = hi;
  a.base = base;
  a.n_base = n_base;
  return FIB_OK;
}

// Calls over several layers with host alphas launch runs of consecutive layers: a run grows
// while the kernel instance picked for its alpha range stays the one its first layer gets
// alone, so no layer runs a wider instance than a single-layer call would (with device
// alphas the host cannot see them, and one launch covers the declared range).
template <typename Args, typename Key>
int64_t run_end(const Args& a, const AlphaArg& al, int64_t s, Key key) {
  Args t = a;
  t.BH = a.heads_per_plan;
  float lo = al.host_list[s], hi = lo;
  t.alpha_lo = t.alpha_hi = lo;
  const int k0 = key(t);
  int64_t e = s + 1;
  for (; e < al.layers; ++e) {
    t.alpha_lo = fminf(lo, al.host_list[e]);
    t.alpha_hi = fmaxf(hi, al.host_list[e]);
    if (key(t) != k0) break;
    lo = t.alpha_lo;
    hi = t.alpha_hi;
  }
  return e;
}

// Args of layers [s, e) of a call over several layers: tensors and plans offset by s layers.
// A run of one layer takes the host-built table as a kernel argument instead (the kernels
// then need not read the plan from memory), i.e. exactly the single-layer call.
template <typename Args>
Args layer_run(const Args& a, const AlphaArg& al, const int32_t* base, int n_base, int64_t s, int64_t e) {
  Args b = a;
  const int64_t hpp = a.heads_per_plan;
  const size_t rows = (size_t)(s * hpp) * (size_t)a.N;
  const size_t bytes = rows * kD * (a.dtype == 0 ? 4 : 2);
  auto off = [&](auto p) { return p == nullptr ? p : (decltype(p))((const char*)p + bytes); };
  b.q = off(a.q);
  b.k = off(a.k);
  b.v = off(a.v);
  if (a.lse != nullptr) b.lse = a.lse + rows;
  if constexpr (std::is_same_v<Args, BwdArgs>) {
    b.o = off(a.o);
    b.dout = off(a.dout);
    b.dq = off(a.dq);
    b.dk = off(a.dk);
    b.dv = off(a.dv);
    if (a.dalpha != nullptr) b.dalpha = a.dalpha + s;
  } else {
    b.o = off(a.o);
  }
  b.plan = a.plan + s;
  b.BH = (e - s) * hpp;
  b.layers = (int)(e - s);
  b.alpha_lo = b.alpha_hi = al.host_list[s];
  for (int64_t l = s; l < e; ++l) {
    b.alpha_lo = fminf(b.alpha_lo, al.host_list[l]);
    b.alpha_hi = fmaxf(b.alpha_hi, al.host_list[l]);
  }
  if (e - s == 1) {
    b.plan = nullptr;
    b.heads_per_plan = 0x7fffffff;
    build_table(al.host_list[s], base, n_base, a.W, a.mode, &b.tab);
  }
  return b;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
             int64_t D, int dtype, int W, const AlphaArg& al, const int32_t* base, int n_base, float rope_theta,
             int mode, void* stream, bool decode) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FIB_ERR_NULL;
  int st = check_shape(B, H, N, D, dtype);
  if (st) return st;
  st = check_base(base, n_base);
  if (st) return st;
  st = check_scalars(W, 1.f, rope_theta, mode);
  if (st) return st;
  st = check_alpha(al);
  if (st) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
    return FIB_ERR_ALIGN;
  FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.BH = B * H; a.N = N; a.dtype = dtype; a.mode = mode; a.W = W;
  a.rope = make_rope(rope_theta);
  a.stream = (hipStream_t)stream;
  st = set_table(a, al, base, n_base);
  if (st) return st;
  auto launch = [&](const FwdArgs& b) {
    if (decode) return launch_decode(b);
    if (fwd_ring_supported(b)) return launch_fwd_ring(b);
    return fwd_gather_preferred(b) ? launch_fwd_gather(b) : launch_fwd_generic(b);
  };
  // (the decode kernel is one instance for every table: one launch serves any stack)
  if (decode || al.dev || al.host_list == nullptr || al.layers == 1)
    return launch(a) == hipSuccess ? FIB_OK : FIB_ERR_LAUNCH;
  for (int64_t s0 = 0; s0 < al.layers;) {
    const int64_t e0 = run_end(a, al, s0, [](const FwdArgs& t) { return fwd_instance_key(t); });
    if (launch(layer_run(a, al, base, n_base, s0, e0)) != hipSuccess) return FIB_ERR_LAUNCH;
    s0 = e0;
  }
  return FIB_OK;
}

// Every argument check of a backward call except the workspace's.
int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
              void* dq, void* dk, void* dv, float* dalpha, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
              int W, const AlphaArg& al, const int32_t* base, int n_base, float rope_theta, int mode) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return FIB_ERR_NULL;
  int st = check_shape(B, H, N, D, dtype);
  if (st) return st;
  st = check_base(base, n_base);
  if (st) return st;
  st = check_scalars(W, 1.f, rope_theta, mode);
  if (st) return st;
  st = check_alpha(al);
  if (st) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u) || ((uintptr_t)dalpha & 3u))
    return FIB_ERR_ALIGN;
  return FIB_OK;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, float* dalpha, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
             int W, const AlphaArg& al, const int32_t* base, int n_base, float rope_theta, int mode,
             void* workspace, size_t workspace_bytes, void* stream) {
  const int st0 = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, dalpha, B, H, N, D, dtype, W, al, base, n_base,
                            rope_theta, mode);
  if (st0) return st0;
  int st;
  const int ps_slots = ps_entry_slots(alpha_max(al), base, n_base, W);
  const size_t need = bwd_workspace_bytes(B * H, N, dtype, mode, ps_slots);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FIB_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned16(workspace)) return FIB_ERR_ALIGN;
  BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dalpha = dalpha;
  a.BH = B * H; a.N = N; a.dtype = dtype; a.mode = mode; a.W = W;
  a.rope = make_rope(rope_theta);
  a.workspace = workspace;
  a.ps_slots = ps_slots;
  a.stream = (hipStream_t)stream;
  st = set_table(a, al, base, n_base);
  if (st) return st;
  if (al.dev || al.host_list == nullptr || al.layers == 1) return launch_bwd(a) == hipSuccess ? FIB_OK : FIB_ERR_LAUNCH;
  // runs share the workspace: they execute one after another on the stream
  for (int64_t s0 = 0; s0 < al.layers;) {
    const int64_t e0 = run_end(a, al, s0, [](const BwdArgs& t) {
      return bwdq_instance_key(t) * 1000 + bwdk_instance_key(t);
    });
    if (launch_bwd(layer_run(a, al, base, n_base, s0, e0)) != hipSuccess) return FIB_ERR_LAUNCH;
    s0 = e0;
  }
  return FIB_OK;
}

AlphaArg host_alpha(float alpha) { return AlphaArg{false, alpha, nullptr, nullptr, 1, 0.f, 0.f, nullptr, 0}; }
AlphaArg dev_alpha(const float* alpha, float lo, float hi, void* plan, size_t plan_bytes, int64_t layers = 1) {
  return AlphaArg{true, 0.f, alpha, nullptr, layers, lo, hi, plan, plan_bytes};
}
AlphaArg host_alphas(const float* alpha, int64_t layers, void* plan, size_t plan_bytes) {
  return AlphaArg{false, 0.f, nullptr, alpha, layers, 0.f, 0.f, plan, plan_bytes};
}

// [L, B, H, N, D] inputs are L * B batches of the single-layer shape
int64_t layer_batches(int64_t L, int64_t B) {
  return (L < 1 || L > kMaxLayers || B < 1 || B > (1LL << 31)) ? 0 : L * B;
}

}  // namespace

extern "C" {

int fib_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                        int W, float alpha, const int32_t* base, int n_base,
                        float rope_theta, int mode, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, D, dtype, W, host_alpha(alpha), base, n_base, rope_theta, mode, stream,
                  false);
}

int fib_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                           int W, float alpha, const int32_t* base, int n_base,
                           float rope_theta, int mode, void* stream) {
  return fwd_impl(q, k_cache, v_cache, o, lse, B, H, N, D, dtype, W, host_alpha(alpha), base, n_base, rope_theta,
                  mode, stream, true);
}

size_t fib_sparse_attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int mode) {
  if (check_shape(B, H, N, D, dtype) != FIB_OK) return 0;
  if (mode != FIB_INT && mode != FIB_INTERP) return 0;
  return bwd_workspace_bytes(B * H, N, dtype, mode, kMaxEnt);
}

size_t fib_sparse_attn_bwd_workspace_size_for(int64_t B, int64_t H, int64_t N, int64_t D, int dtype, int mode,
                                              int W, float alpha_max, const int32_t* base, int n_base) {
  if (check_shape(B, H, N, D, dtype) != FIB_OK) return 0;
  if (mode != FIB_INT && mode != FIB_INTERP) return 0;
  if (check_base(base, n_base) != FIB_OK || W < 1 || !isfinite(alpha_max) || alpha_max <= 0.f) return 0;
  return bwd_workspace_bytes(B * H, N, dtype, mode, ps_entry_slots(alpha_max, base, n_base, W));
}

int fib_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse,
                        void* dq, void* dk, void* dv, float* dalpha,
                        int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                        int W, float alpha, const int32_t* base, int n_base,
                        float rope_theta, int mode,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, dalpha, B, H, N, D, dtype, W, host_alpha(alpha), base, n_base,
                  rope_theta, mode, workspace, workspace_bytes, stream);
}

int fib_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse,
                                void* dq, void* dk, void* dv, float* dalpha,
                                int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                int W, float alpha, const int32_t* base, int n_base,
                                float rope_theta, int mode, void* stream) {
  const int st0 = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, dalpha, B, H, N, D, dtype, W, host_alpha(alpha), base,
                            n_base, rope_theta, mode);
  if (st0) return st0;
  const size_t need = fib_sparse_attn_bwd_workspace_size_for(B, H, N, D, dtype, mode, W, alpha, base, n_base);
  if (need == 0 || need > kScratchBytes) return FIB_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != FIB_OK) return st;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, dalpha, B, H, N, D, dtype, W, host_alpha(alpha), base, n_base,
                  rope_theta, mode, ws, kScratchBytes, stream);
}

size_t fib_dense_lse_workspace_size(int64_t B, int64_t H, int64_t N, int64_t D, int dtype) {
  if (check_shape(B, H, N, D, dtype) != FIB_OK) return 0;
  return dense_lse_workspace_bytes(B * H, N);
}

int fib_dense_causal_lse(const void* q, const void* k, float* lse, int64_t B, int64_t H, int64_t N, int64_t D,
                         int dtype, float rope_theta, void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || k == nullptr || lse == nullptr) return FIB_ERR_NULL;
  int st = check_shape(B, H, N, D, dtype);
  if (st) return st;
  if (!isfinite(rope_theta) || rope_theta <= 0.f) return FIB_ERR_THETA;
  if ((double)(B * H) * (double)((N + 127) / 128) > 2147483647.0) return FIB_ERR_SHAPE;
  if (workspace == nullptr || workspace_bytes < dense_lse_workspace_bytes(B * H, N)) return FIB_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(workspace) || ((uintptr_t)lse & 3u)) return FIB_ERR_ALIGN;
  return launch_dense_lse(q, k, lse, B * H, N, dtype, make_rope(rope_theta), workspace, (hipStream_t)stream) ==
                 hipSuccess
             ? FIB_OK
             : FIB_ERR_LAUNCH;
}

int fib_sparse_attn_dropped_mass(const float* lse_sparse, const float* lse_dense, float* dropped, int64_t count,
                                 void* stream) {
  if (lse_sparse == nullptr || lse_dense == nullptr || dropped == nullptr) return FIB_ERR_NULL;
  if (count < 1 || count > (1LL << 40)) return FIB_ERR_SHAPE;
  if (((uintptr_t)lse_sparse & 3u) || ((uintptr_t)lse_dense & 3u) || ((uintptr_t)dropped & 3u)) return FIB_ERR_ALIGN;
  return launch_dropped_mass(lse_sparse, lse_dense, dropped, count, (hipStream_t)stream) == hipSuccess
             ? FIB_OK
             : FIB_ERR_LAUNCH;
}

size_t fib_sparse_attn_plan_bytes(void) { return sizeof(DevPlan); }

size_t fib_sparse_attn_layers_plan_bytes(int64_t n_layers) {
  return n_layers < 1 || n_layers > kMaxLayers ? 0 : (size_t)n_layers * sizeof(DevPlan);
}

int fib_sparse_attn_fwd_layers(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, const int32_t* base, int n_base,
                               float rope_theta, int mode, void* plan, size_t plan_bytes, void* stream) {
  if (alpha == nullptr) return FIB_ERR_NULL;
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return fwd_impl(q, k, v, o, lse, LB, H, N, D, dtype, W, host_alphas(alpha, L, plan, plan_bytes), base, n_base,
                  rope_theta, mode, stream, false);
}

int fib_sparse_attn_decode_layers(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                  int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                  int W, const float* alpha, const int32_t* base, int n_base,
                                  float rope_theta, int mode, void* plan, size_t plan_bytes, void* stream) {
  if (alpha == nullptr) return FIB_ERR_NULL;
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return fwd_impl(q, k_cache, v_cache, o, lse, LB, H, N, D, dtype, W, host_alphas(alpha, L, plan, plan_bytes), base,
                  n_base, rope_theta, mode, stream, true);
}

int fib_sparse_attn_decode_layers_dev(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                      int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                      int W, const float* alpha, float alpha_lo, float alpha_hi,
                                      const int32_t* base, int n_base, float rope_theta, int mode,
                                      void* plan, size_t plan_bytes, void* stream) {
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return fwd_impl(q, k_cache, v_cache, o, lse, LB, H, N, D, dtype, W,
                  dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes, L), base, n_base, rope_theta, mode, stream,
                  true);
}

int fib_sparse_attn_fwd_layers_dev(const void* q, const void* k, const void* v, void* o, float* lse,
                                   int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                   int W, const float* alpha, float alpha_lo, float alpha_hi,
                                   const int32_t* base, int n_base, float rope_theta, int mode,
                                   void* plan, size_t plan_bytes, void* stream) {
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return fwd_impl(q, k, v, o, lse, LB, H, N, D, dtype, W, dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes, L),
                  base, n_base, rope_theta, mode, stream, false);
}

int fib_sparse_attn_bwd_layers(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse,
                               void* dq, void* dk, void* dv, float* dalpha,
                               int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, const int32_t* base, int n_base,
                               float rope_theta, int mode, void* workspace, size_t workspace_bytes,
                               void* plan, size_t plan_bytes, void* stream) {
  if (alpha == nullptr) return FIB_ERR_NULL;
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, dalpha, LB, H, N, D, dtype, W,
                  host_alphas(alpha, L, plan, plan_bytes), base, n_base, rope_theta, mode, workspace,
                  workspace_bytes, stream);
}

int fib_sparse_attn_bwd_layers_dev(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse,
                                   void* dq, void* dk, void* dv, float* dalpha,
                                   int64_t L, int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                                   int W, const float* alpha, float alpha_lo, float alpha_hi,
                                   const int32_t* base, int n_base, float rope_theta, int mode,
                                   void* workspace, size_t workspace_bytes, void* plan, size_t plan_bytes,
                                   void* stream) {
  const int64_t LB = layer_batches(L, B);
  if (LB == 0) return FIB_ERR_SHAPE;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, dalpha, LB, H, N, D, dtype, W,
                  dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes, L), base, n_base, rope_theta, mode,
                  workspace, workspace_bytes, stream);
}

int fib_sparse_attn_fwd_dev(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                            int W, const float* alpha, float alpha_lo, float alpha_hi,
                            const int32_t* base, int n_base, float rope_theta, int mode,
                            void* plan, size_t plan_bytes, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, D, dtype, W, dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes),
                  base, n_base, rope_theta, mode, stream, false);
}

int fib_sparse_attn_decode_dev(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                               int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                               int W, const float* alpha, float alpha_lo, float alpha_hi,
                               const int32_t* base, int n_base, float rope_theta, int mode,
                               void* plan, size_t plan_bytes, void* stream) {
  return fwd_impl(q, k_cache, v_cache, o, lse, B, H, N, D, dtype, W,
                  dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes), base, n_base, rope_theta, mode, stream,
                  true);
}

int fib_sparse_attn_bwd_dev(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse,
                            void* dq, void* dk, void* dv, float* dalpha,
                            int64_t B, int64_t H, int64_t N, int64_t D, int dtype,
                            int W, const float* alpha, float alpha_lo, float alpha_hi,
                            const int32_t* base, int n_base, float rope_theta, int mode,
                            void* workspace, size_t workspace_bytes, void* plan, size_t plan_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, dalpha, B, H, N, D, dtype, W,
                  dev_alpha(alpha, alpha_lo, alpha_hi, plan, plan_bytes), base, n_base, rope_theta, mode, workspace,
                  workspace_bytes, stream);
}

}  // extern "C"
