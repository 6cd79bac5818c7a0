// alpha held in device memory: the launch data that depends on alpha (the offset table and
// its ring splits) is built on the device, so a call needs no host copy of alpha and no
// stream synchronization (the Learned schedule of "Depth-Staggered Fibonacci Spacing for
// Sparse Attention", Method > Experimental variables, trains alpha on the device).
//
// The host picks kernel instances from an alpha range [lo, hi] (range_counts bounds the
// covered and far counts over it); one thread builds the table and splits from the clamped
// alpha with the same code as the host path (build_table, make_split).
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

__global__ void dev_plan_kernel(DevPlan* out, const float* alpha, float lo, float hi, BaseList base, int n_base, int W,
                                int mode, int64_t N) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  // clamped into the range the launch was planned for (a NaN becomes lo)
  const float a = fminf(fmaxf(*alpha, lo), hi);
  build_table(a, base.v, n_base, W, mode, &out->tab);
  make_split(out->tab, N, 8, mode, &out->s8);
  make_split(out->tab, N, 4, mode, &out->s4);
}

}  // namespace

hipError_t launch_dev_plan(DevPlan* out, const float* alpha, float lo, float hi, const BaseList& base, int n_base,
                           int W, int mode, int64_t N, hipStream_t s) {
  dev_plan_kernel<<<1, 64, 0, s>>>(out, alpha, lo, hi, base, n_base, W, mode, N);
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
