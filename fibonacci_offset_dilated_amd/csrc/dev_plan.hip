// alpha held in device memory: the launch data that depends on alpha (the offset table and
// its ring splits) is built on the device, so a call needs no host copy of alpha and no
// stream synchronization (the Learned schedule of "Depth-Staggered Fibonacci Spacing for
// Sparse Attention", Method > Experimental variables, trains alpha on the device).
//
// The host picks kernel instances from an alpha range [lo, hi] (range_counts bounds the
// covered and far counts over it); one wave per layer builds the table and splits from the
// clamped alpha by the rules of the host path (build_table, make_split). The same
// plans serve calls over several layers at once (one alpha per layer, from device memory or
// passed by value from the host).
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

// One wave per layer. The table and its splits are what build_table and make_split give on
// the host (the same fp64 products, rint and ceil, the same keep, collapse and split rules),
// computed lane-parallel: lane e evaluates base entry e, ballots give the kept set and each
// entry's slot, and the sorted table (distances are non-decreasing in f in both modes) makes
// every count a popcount and every maximum the last entry of a prefix. A single lane running
// the serial builders takes ~10 us on its dependent reads.
__global__ __launch_bounds__(64) void dev_plan_kernel(DevPlan* out, const float* alpha, AlphaList host, int L,
                                                      float lo, float hi, BaseList base, int n_base, int W, int mode,
                                                      int64_t N) {
  static_assert(sizeof(DevPlan) % 4 == 0, "plan is copied in 32-bit words");
  static_assert(kMaxEnt <= 32, "one lane per base entry, masks in 32 bits");
  __shared__ DevPlan p;
  const int l = blockIdx.x;
  if (l >= L) return;
  const int e = threadIdx.x;
  // a device alpha is clamped into the range the launch was planned for (a NaN becomes lo)
  const float a = alpha != nullptr ? fminf(fmaxf(alpha[l], lo), hi) : host.v[l];

  // ---- the table
  const bool valid = e < n_base;
  const int32_t f = valid ? base.v[e < kMaxEnt ? e : 0] : 0;
  const double d = (double)a * (double)f;
  bool keep;
  int dist = 0;
  float w = 0.f;
  if (mode == 0) {
    const double r = rint(d);
    keep = valid && r >= (double)W && r <= 2147483647.0;
    dist = keep ? (int)r : 0;
  } else {
    const double c = ceil(d);
    keep = valid && d >= (double)W && c <= 2147483647.0;
    dist = keep ? (int)c : 0;
    w = keep ? (float)(c - d) : 0.f;
  }
  const uint32_t below = (1u << (e & 31)) - 1u;  // lanes e' < e (e < 32)
  uint32_t kept = (uint32_t)__ballot(keep);
  if (mode == 0) {
    // equal offsets collapse: drop an entry equal to the previous kept one
    const uint32_t prev = kept & below;
    const int pl = prev ? 31 - __builtin_clz(prev) : 0;
    const int pd = __shfl(dist, pl);
    const bool dup = keep && prev != 0 && pd == dist;
    kept = (uint32_t)__ballot(keep && !dup);
    keep = keep && !dup;
  }
  const int n_ent = __builtin_popcount(kept);
  if (e < kMaxEnt) {
    p.tab.dist[e] = 0;
    p.tab.w[e] = 0.f;
    p.tab.f[e] = 0.f;
  }
  __syncthreads();
  if (keep) {
    const int slot = __builtin_popcount(kept & below);
    p.tab.dist[slot] = dist;
    p.tab.w[slot] = w;
    p.tab.f[slot] = mode == 1 ? (float)f : 0.f;
  }
  if (e == 0) p.tab.n = n_ent;
  __syncthreads();

  // ---- ring splits for 8 and 4 waves (as make_split)
  const int usable = __builtin_popcount((uint32_t)__ballot(keep && (int64_t)dist < N));
  for (int v = 0; v < 2; ++v) {
    const int waves = v == 0 ? 8 : 4;
    RingSplit& sp = v == 0 ? p.s8 : p.s4;
    const int reach = ring_reach(waves);
    const int cov = __builtin_popcount((uint32_t)__ballot(keep && (int64_t)dist < N && dist <= reach));
    if (e == 0) {
      sp.n_cov = cov;
      sp.n_far = usable - cov;
      sp.need = cov > 0 && p.tab.dist[cov - 1] > kBandRows ? p.tab.dist[cov - 1] : kBandRows;
      sp.early_rows = usable > 0 && p.tab.dist[usable - 1] > kBandRows ? p.tab.dist[usable - 1] : kBandRows;
    }
    if (e < kSplitCov) {
      const bool use = e < cov;
      sp.dist[e] = use ? p.tab.dist[e] : kBandRows;
      sp.w[e] = use ? p.tab.w[e] : 0.f;
      sp.f[e] = use ? p.tab.f[e] : 0.f;
    }
    if (e < kSplitFar) {
      const bool use = e < usable - cov && cov + e < kMaxEnt;
      const int fd = use ? p.tab.dist[cov + e] : reach + 1;
      sp.far_dist[e] = fd;
      sp.far_w[e] = use ? p.tab.w[cov + e] : 0.f;
      sp.far_f[e] = use ? p.tab.f[cov + e] : 0.f;
      if (mode == 1) {
        sp.unc_dist[2 * e] = fd;
        sp.unc_dist[2 * e + 1] = fd - 1;
      } else {
        sp.unc_dist[e] = fd;
        sp.unc_dist[kSplitFar + e] = 0;
      }
    }
  }
  __syncthreads();
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&p);
  uint32_t* dst = reinterpret_cast<uint32_t*>(out + l);
  for (int x = threadIdx.x; x < (int)(sizeof(DevPlan) / 4); x += 64) dst[x] = src[x];
}

}  // namespace

hipError_t launch_dev_plan(DevPlan* out, const float* alpha, const AlphaList& host, int L, float lo, float hi,
                           const BaseList& base, int n_base, int W, int mode, int64_t N, hipStream_t s) {
  dev_plan_kernel<<<L, 64, 0, s>>>(out, alpha, host, L, lo, hi, base, n_base, W, mode, N);
  return hipGetLastError();
}

// An entry can be covered for some alpha in [lo, hi] when it is kept at hi (distances grow
// with alpha) and within the ring's reach at lo; it can be far when it is beyond the reach at
// hi and usable (distance < N) at lo. Counting entries independently bounds the prefix
// counts of make_split (integer-mode collapsing only lowers them).
void range_counts(float lo, float hi, const int32_t* base, int n_base, int W, int mode, int64_t N, int waves,
                  int* n_cov, int* n_far) {
  const int reach = ring_reach(waves);
  int cov = 0, far = 0;
  for (int e = 0; e < n_base; ++e) {
    const double dl = (double)lo * (double)base[e], dh = (double)hi * (double)base[e];
    const double kl = mode == 0 ? rint(dl) : ceil(dl);
    const double kh = mode == 0 ? rint(dh) : ceil(dh);
    const bool kept = mode == 0 ? kh >= (double)W : dh >= (double)W;
    if (!kept || kl >= (double)N) continue;
    if (kl <= (double)reach) ++cov;
    if (kh > (double)reach) ++far;
  }
  *n_cov = cov;
  *n_far = far;
}

}  // namespace fib
