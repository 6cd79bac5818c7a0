// Backward of Fibonacci-offset dilated sparse attention: dQ, dK, dV and d(alpha).
//
// Source: "Depth-Staggered Fibonacci Spacing for Sparse Attention" (gist.science summaries
// of arXiv 2606.28560), Method > Architecture and attention mechanism: the interpolation of
// key/value rows at non-integer offsets exists so that the gradient reaches alpha (the
// Learned schedule of Method > Experimental variables trains alpha by gradient descent).
//
// With s = <R_i q_i, R_j k_j>/sqrt(D) = <R_(i-j) q_i, k_j>/sqrt(D), P = exp(s - LSE_i),
// Delta_i = <dO_i, O_i>, dP = <dO_i, value>, dS = P (dP - Delta_i):
//   dQ_i  = sum_k dS_ik R_(i-j)^T k_j / sqrt(D)        (gradient w.r.t. the un-rotated q)
//   dK_j += weight * dS_ik R_(i-j) q_i / sqrt(D)       (gradient w.r.t. the un-rotated k)
//   dV_j += weight * P_ik dO_i
// where weight is 1 for window and integer keys and (1 - w) / w on the lower / upper row of an
// interpolated key. With w = c - alpha f, dw/dalpha = -f:
//   dalpha = sum_ik -f_k [dS_ik (s_hi - s_lo) + P_ik <dO_i, v_hi - v_lo>]
// with s_lo = <R_c q_i, k_lo>/sqrt(D), s_hi = <R_(c-1) q_i, k_hi>/sqrt(D).
//
// Three deterministic kernels (no floating-point atomics):
//   1. query-side: per query, recompute the logits, write dQ and Delta, and a per-block
//      partial of dalpha;
//   2. key-side: per key row j, gather every (query, key) pair that reads row j (window
//      queries j..j+W-1, integer offsets j + r, interpolated lower-row queries j + c and
//      upper-row queries j + c - 1) and accumulate dK_j, dV_j in registers;
//   3. a single block sums the dalpha partials in a fixed order.
// Lane layout as in the general forward kernel: a quad of 4 lanes per row, 16 dims per lane.
// For bf16 with W <= 16 the query and key sides run on the LDS-ring kernels of bwd_ring.hip
// and bwd_key_ring.hip instead (run() below picks them); this file also holds the workspace
// layout and the key side that reads the interpolated (P, dS) words when the ring key side
// does not apply (more than 3 far entries).
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

constexpr int kRPB = 64;  // rows per block

template <typename T, int MODE, bool DEV>
__global__ __launch_bounds__(256) void bwd_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
    const T* __restrict__ dout, const float* __restrict__ lse, T* __restrict__ dq, float* __restrict__ delta,
    float* __restrict__ dalpha_part, int64_t N, int W, Table tab_arg, Rope rope, float scale, int tiles,
    const DevPlan* __restrict__ plan, int heads_per_plan) {
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)(blockIdx.x / tiles) / heads_per_plan);
  __shared__ float2 cs[kCsSlots][kHalf];
  __shared__ float red[256];
  const bool cached = fill_cs(cs, W, tab, MODE, rope);
  const int64_t head = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int c = threadIdx.x & 3;
  const int64_t i = (int64_t)tile * kRPB + (threadIdx.x >> 2);
  const bool active = i < N;
  const int64_t ii = active ? i : N - 1;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const T* kh_ = k + hoff;
  const T* vh_ = v + hoff;
  const float log2e = 1.4426950408889634f;

  float ql[8], qh[8], dol[8], doh[8], ol[8], oh[8];
  Vec8<T>::load(q + hoff + ii * kD + 8 * c, ql);
  Vec8<T>::load(q + hoff + ii * kD + kHalf + 8 * c, qh);
  Vec8<T>::load(dout + hoff + ii * kD + 8 * c, dol);
  Vec8<T>::load(dout + hoff + ii * kD + kHalf + 8 * c, doh);
  Vec8<T>::load(o + hoff + ii * kD + 8 * c, ol);
  Vec8<T>::load(o + hoff + ii * kD + kHalf + 8 * c, oh);
  const float dlt = quad_sum(dot16(dol, doh, ol, oh));
  const float lse2 = lse[(size_t)head * N + ii] * log2e;
  const float sl2 = scale * log2e;

  float gl[8], gh[8];  // dQ accumulator (lane's 16 dims)
#pragma unroll
  for (int t = 0; t < 8; ++t) gl[t] = gh[t] = 0.f;
  float dal = 0.f;

  // dQ += g * R_dist^T x for the lane's pairs (rotation by -dist)
  auto add_rot_t = [&](float g, const float* xl, const float* xh, int slot, int64_t dist) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 a = get_cs(cs, cached, slot, dist, 8 * c + t, rope);
      gl[t] = fmaf(g, xl[t] * a.x + xh[t] * a.y, gl[t]);
      gh[t] = fmaf(g, xh[t] * a.x - xl[t] * a.y, gh[t]);
    }
  };

  float kl[8], kh[8], vl[8], vh[8], rl[8], rh[8];
  const int64_t wmax = (int64_t)W < ii + 1 ? (int64_t)W : ii + 1;
  for (int64_t s = 0; s < wmax; ++s) {
    const int64_t j = ii - s;
    Vec8<T>::load(kh_ + j * kD + 8 * c, kl);
    Vec8<T>::load(kh_ + j * kD + kHalf + 8 * c, kh);
    Vec8<T>::load(vh_ + j * kD + 8 * c, vl);
    Vec8<T>::load(vh_ + j * kD + kHalf + 8 * c, vh);
    rotate8(ql, qh, rl, rh, cs, cached, (int)s, s, c, rope);
    const float sc = quad_sum(dot16(rl, rh, kl, kh));
    const float p = exp2f(sc * sl2 - lse2);
    const float dp = quad_sum(dot16(dol, doh, vl, vh));
    add_rot_t(p * (dp - dlt) * scale, kl, kh, (int)s, s);
  }
  for (int e = 0; e < tab.n; ++e) {
    int64_t lo;
    if (!entry_row(tab, e, ii, &lo)) continue;
    const int64_t d = tab.dist[e];
    Vec8<T>::load(kh_ + lo * kD + 8 * c, kl);
    Vec8<T>::load(kh_ + lo * kD + kHalf + 8 * c, kh);
    Vec8<T>::load(vh_ + lo * kD + 8 * c, vl);
    Vec8<T>::load(vh_ + lo * kD + kHalf + 8 * c, vh);
    rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
    const float s_lo = quad_sum(dot16(rl, rh, kl, kh));
    const float dp_lo = quad_sum(dot16(dol, doh, vl, vh));
    if (MODE == 0) {
      const float p = exp2f(s_lo * sl2 - lse2);
      add_rot_t(p * (dp_lo - dlt) * scale, kl, kh, W + e, d);
    } else {
      const float w = tab.w[e];
      float kl2[8], kh2[8], vl2[8], vh2[8];
      Vec8<T>::load(kh_ + (lo + 1) * kD + 8 * c, kl2);
      Vec8<T>::load(kh_ + (lo + 1) * kD + kHalf + 8 * c, kh2);
      Vec8<T>::load(vh_ + (lo + 1) * kD + 8 * c, vl2);
      Vec8<T>::load(vh_ + (lo + 1) * kD + kHalf + 8 * c, vh2);
      rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
      const float s_hi = quad_sum(dot16(rl, rh, kl2, kh2));
      const float dp_hi = quad_sum(dot16(dol, doh, vl2, vh2));
      const float sc = fmaf(w, s_hi - s_lo, s_lo);
      const float p = exp2f(sc * sl2 - lse2);
      const float dp = fmaf(w, dp_hi - dp_lo, dp_lo);
      const float ds = p * (dp - dlt);
      add_rot_t(ds * scale * (1.f - w), kl, kh, W + e, d);
      add_rot_t(ds * scale * w, kl2, kh2, W + tab.n + e, d - 1);
      dal = fmaf(-tab.f[e], ds * scale * (s_hi - s_lo) + p * (dp_hi - dp_lo), dal);
    }
  }
  if (active) {
    Vec8<T>::store(dq + hoff + i * kD + 8 * c, gl);
    Vec8<T>::store(dq + hoff + i * kD + kHalf + 8 * c, gh);
    if (c == 0) delta[(size_t)head * N + i] = dlt;
  }
  if (MODE == 1) {
    // per-block partial of dalpha: one value per query (lane c == 0), fixed-order tree
    red[threadIdx.x] = (active && c == 0) ? dal : 0.f;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
      __syncthreads();
    }
    if (threadIdx.x == 0) dalpha_part[blockIdx.x] = red[0];
  }
}

template <typename T, int MODE, bool DEV>
__global__ __launch_bounds__(256) void bwd_key_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, T* __restrict__ dk, T* __restrict__ dv,
    int64_t N, int W, Table tab_arg, Rope rope, float scale, int tiles, const DevPlan* __restrict__ plan,
    int heads_per_plan) {
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)(blockIdx.x / tiles) / heads_per_plan);
  __shared__ float2 cs[kCsSlots][kHalf];
  const bool cached = fill_cs(cs, W, tab, MODE, rope);
  const int64_t head = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int c = threadIdx.x & 3;
  const int64_t j = (int64_t)tile * kRPB + (threadIdx.x >> 2);
  const bool active = j < N;
  const int64_t jj = active ? j : N - 1;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const T* qh_ = q + hoff;
  const T* kh_ = k + hoff;
  const T* vh_ = v + hoff;
  const T* doh_ = dout + hoff;
  const float* lse_h = lse + (size_t)head * N;
  const float* dlt_h = delta + (size_t)head * N;
  const float log2e = 1.4426950408889634f;
  const float sl2 = scale * log2e;

  float kl[8], kh[8], vl[8], vh[8];
  Vec8<T>::load(kh_ + jj * kD + 8 * c, kl);
  Vec8<T>::load(kh_ + jj * kD + kHalf + 8 * c, kh);
  Vec8<T>::load(vh_ + jj * kD + 8 * c, vl);
  Vec8<T>::load(vh_ + jj * kD + kHalf + 8 * c, vh);

  float akl[8], akh[8], avl[8], avh[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) akl[t] = akh[t] = avl[t] = avh[t] = 0.f;

  float ql[8], qh[8], dol[8], doh[8], rl[8], rh[8];
  auto load_query = [&](int64_t i) {
    Vec8<T>::load(qh_ + i * kD + 8 * c, ql);
    Vec8<T>::load(qh_ + i * kD + kHalf + 8 * c, qh);
    Vec8<T>::load(doh_ + i * kD + 8 * c, dol);
    Vec8<T>::load(doh_ + i * kD + kHalf + 8 * c, doh);
  };
  // accumulate weight * (dS * scale * R_dist q_i, P * dO_i); rl/rh hold R_dist q_i
  auto accum = [&](float gk, float gv) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      akl[t] = fmaf(gk, rl[t], akl[t]);
      akh[t] = fmaf(gk, rh[t], akh[t]);
      avl[t] = fmaf(gv, dol[t], avl[t]);
      avh[t] = fmaf(gv, doh[t], avh[t]);
    }
  };

  // window queries i = j + s and integer-offset queries i = j + r: key row j itself
  const int64_t wmax = (int64_t)W < N - jj ? (int64_t)W : N - jj;
  for (int64_t s = 0; s < wmax; ++s) {
    const int64_t i = jj + s;
    load_query(i);
    rotate8(ql, qh, rl, rh, cs, cached, (int)s, s, c, rope);
    const float sc = quad_sum(dot16(rl, rh, kl, kh));
    const float p = exp2f(sc * sl2 - lse_h[i] * log2e);
    const float dp = quad_sum(dot16(dol, doh, vl, vh));
    accum(p * (dp - dlt_h[i]) * scale, p);
  }
  for (int e = 0; e < tab.n; ++e) {
    const int64_t d = tab.dist[e];
    if (MODE == 0) {
      const int64_t i = jj + d;
      if (i >= N) continue;
      load_query(i);
      rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
      const float sc = quad_sum(dot16(rl, rh, kl, kh));
      const float p = exp2f(sc * sl2 - lse_h[i] * log2e);
      const float dp = quad_sum(dot16(dol, doh, vl, vh));
      accum(p * (dp - dlt_h[i]) * scale, p);
    } else {
      const float w = tab.w[e];
      // row j as the lower row (distance c) of query i = j + c; upper row j + 1
      {
        const int64_t i = jj + d;
        if (i < N) {
          load_query(i);
          float k2l[8], k2h[8], v2l[8], v2h[8];
          Vec8<T>::load(kh_ + (jj + 1) * kD + 8 * c, k2l);
          Vec8<T>::load(kh_ + (jj + 1) * kD + kHalf + 8 * c, k2h);
          Vec8<T>::load(vh_ + (jj + 1) * kD + 8 * c, v2l);
          Vec8<T>::load(vh_ + (jj + 1) * kD + kHalf + 8 * c, v2h);
          rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
          const float s_hi = quad_sum(dot16(rl, rh, k2l, k2h));
          const float dp_hi = quad_sum(dot16(dol, doh, v2l, v2h));
          rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
          const float s_lo = quad_sum(dot16(rl, rh, kl, kh));
          const float dp_lo = quad_sum(dot16(dol, doh, vl, vh));
          const float p = exp2f(fmaf(w, s_hi - s_lo, s_lo) * sl2 - lse_h[i] * log2e);
          const float ds = p * (fmaf(w, dp_hi - dp_lo, dp_lo) - dlt_h[i]);
          accum(ds * scale * (1.f - w), p * (1.f - w));
        }
      }
      // row j as the upper row (distance c - 1) of query i = j + c - 1; lower row j - 1
      {
        const int64_t i = jj + d - 1;
        if (i < N && jj >= 1) {
          load_query(i);
          float k0l[8], k0h[8], v0l[8], v0h[8];
          Vec8<T>::load(kh_ + (jj - 1) * kD + 8 * c, k0l);
          Vec8<T>::load(kh_ + (jj - 1) * kD + kHalf + 8 * c, k0h);
          Vec8<T>::load(vh_ + (jj - 1) * kD + 8 * c, v0l);
          Vec8<T>::load(vh_ + (jj - 1) * kD + kHalf + 8 * c, v0h);
          rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
          const float s_lo = quad_sum(dot16(rl, rh, k0l, k0h));
          const float dp_lo = quad_sum(dot16(dol, doh, v0l, v0h));
          rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
          const float s_hi = quad_sum(dot16(rl, rh, kl, kh));
          const float dp_hi = quad_sum(dot16(dol, doh, vl, vh));
          const float p = exp2f(fmaf(w, s_hi - s_lo, s_lo) * sl2 - lse_h[i] * log2e);
          const float ds = p * (fmaf(w, dp_hi - dp_lo, dp_lo) - dlt_h[i]);
          accum(ds * scale * w, p * w);
        }
      }
    }
  }
  if (!active) return;
  Vec8<T>::store(dk + hoff + j * kD + 8 * c, akl);
  Vec8<T>::store(dk + hoff + j * kD + kHalf + 8 * c, akh);
  Vec8<T>::store(dv + hoff + j * kD + 8 * c, avl);
  Vec8<T>::store(dv + hoff + j * kD + kHalf + 8 * c, avh);
}

// Key side in interpolated mode when the query side stored each (query, entry)'s P and dS
// (ps_pack words in ps[(head * ps_slots + e) * N + i]): the window queries are recomputed as in
// bwd_key_kernel; for table entry e (c, w) row j is the lower row of query j + c (weight
// 1 - w) and the upper row of query j + c - 1 (weight w), so
//   dK_j += weight * dS * R_dist q_i / sqrt(D), dV_j += weight * P * dO_i
// with dist = c or c - 1, and no logit of an interpolated key is recomputed.
template <bool DEV>
__global__ __launch_bounds__(256) void bwd_key_ps_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const uint32_t* __restrict__ ps, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int64_t N, int W,
    Table tab_arg, Rope rope, float scale, int tiles, const DevPlan* __restrict__ plan,
    int heads_per_plan, int ps_slots) {
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)(blockIdx.x / tiles) / heads_per_plan);
  __shared__ float2 cs[kCsSlots][kHalf];
  const bool cached = fill_cs(cs, W, tab, 1, rope);
  const int64_t head = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int c = threadIdx.x & 3;
  const int64_t j = (int64_t)tile * kRPB + (threadIdx.x >> 2);
  const bool active = j < N;
  const int64_t jj = active ? j : N - 1;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const bf16_t* qh_ = q + hoff;
  const bf16_t* kh_ = k + hoff;
  const bf16_t* vh_ = v + hoff;
  const bf16_t* doh_ = dout + hoff;
  const float* lse_h = lse + (size_t)head * N;
  const float* dlt_h = delta + (size_t)head * N;
  const float log2e = 1.4426950408889634f;
  const float sl2 = scale * log2e;

  float kl[8], kh[8], vl[8], vh[8];
  Vec8<bf16_t>::load(kh_ + jj * kD + 8 * c, kl);
  Vec8<bf16_t>::load(kh_ + jj * kD + kHalf + 8 * c, kh);
  Vec8<bf16_t>::load(vh_ + jj * kD + 8 * c, vl);
  Vec8<bf16_t>::load(vh_ + jj * kD + kHalf + 8 * c, vh);

  float akl[8], akh[8], avl[8], avh[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) akl[t] = akh[t] = avl[t] = avh[t] = 0.f;

  float ql[8], qh[8], dol[8], doh[8], rl[8], rh[8];
  auto load_query = [&](int64_t i) {
    Vec8<bf16_t>::load(qh_ + i * kD + 8 * c, ql);
    Vec8<bf16_t>::load(qh_ + i * kD + kHalf + 8 * c, qh);
    Vec8<bf16_t>::load(doh_ + i * kD + 8 * c, dol);
    Vec8<bf16_t>::load(doh_ + i * kD + kHalf + 8 * c, doh);
  };
  auto accum = [&](float gk, float gv) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      akl[t] = fmaf(gk, rl[t], akl[t]);
      akh[t] = fmaf(gk, rh[t], akh[t]);
      avl[t] = fmaf(gv, dol[t], avl[t]);
      avh[t] = fmaf(gv, doh[t], avh[t]);
    }
  };

  // window queries i = j + s
  const int64_t wmax = (int64_t)W < N - jj ? (int64_t)W : N - jj;
  for (int64_t s = 0; s < wmax; ++s) {
    const int64_t i = jj + s;
    load_query(i);
    rotate8(ql, qh, rl, rh, cs, cached, (int)s, s, c, rope);
    const float sc = quad_sum(dot16(rl, rh, kl, kh));
    const float p = exp2f(sc * sl2 - lse_h[i] * log2e);
    const float dp = quad_sum(dot16(dol, doh, vl, vh));
    accum(p * (dp - dlt_h[i]) * scale, p);
  }
  // table entries: stored P and dS of the queries that read row j
  for (int e = 0; e < tab.n; ++e) {
    const int64_t d = tab.dist[e];
    const float w = tab.w[e];
    const uint32_t* pse = ps + ((size_t)head * ps_slots + e) * N;
    const int64_t i_lo = jj + d;      // row j is its lower row
    const int64_t i_hi = jj + d - 1;  // row j is its upper row (its lower row j - 1 must exist)
    if (i_lo < N) {
      const uint32_t x = pse[i_lo];
      load_query(i_lo);
      rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
      accum(ps_ds(x) * scale * (1.f - w), ps_p(x) * (1.f - w));
    }
    if (i_hi < N && jj >= 1) {
      const uint32_t x = pse[i_hi];
      load_query(i_hi);
      rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
      accum(ps_ds(x) * scale * w, ps_p(x) * w);
    }
  }
  if (!active) return;
  Vec8<bf16_t>::store(dk + hoff + j * kD + 8 * c, akl);
  Vec8<bf16_t>::store(dk + hoff + j * kD + kHalf + 8 * c, akh);
  Vec8<bf16_t>::store(dv + hoff + j * kD + 8 * c, avl);
  Vec8<bf16_t>::store(dv + hoff + j * kD + kHalf + 8 * c, avh);
}

// Sums n partials in a fixed order (per-thread strided sums, then a tree); block b sums the
// b-th run of n partials (one layer's workgroups) into out[b].
__global__ __launch_bounds__(256) void dalpha_reduce_kernel(const float* __restrict__ part, int64_t n,
                                                            float* __restrict__ out) {
  __shared__ double red[256];
  part += (int64_t)blockIdx.x * n;
  out += blockIdx.x;
  double s = 0.0;
  for (int64_t x = threadIdx.x; x < n; x += 256) s += (double)part[x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = (float)red[0];
}

__global__ void store_zero_kernel(float* out, int n) {
  for (int x = threadIdx.x; x < n; x += blockDim.x) out[x] = 0.f;
}

int64_t tiles_of(int64_t N) { return (N + kRPB - 1) / kRPB; }

// Workspace: Delta [BH * N] fp32 (padded to 64 floats), one d(alpha) partial per query-side
// workgroup (at most BH * tiles_of(N)), 64 spare floats; then, for bf16 inputs in
// interpolated mode, the rotated rows R_i q_i and R_j k_j [BH][N][D] (bf16, 16-byte aligned)
// that the ring query side writes and the (P, dS) words (ps_pack) [BH][ps_slots][N].
size_t rot_offset_bytes(int64_t BH, int64_t N) {
  const size_t floats = (size_t)(((BH * N + 63) / 64) * 64 + BH * tiles_of(N) + 64);
  return ((floats * sizeof(float) + 15) / 16) * 16;
}
size_t rot_bytes(int64_t BH, int64_t N) { return (size_t)BH * (size_t)N * kD * sizeof(bf16_t); }
size_t ps_offset_bytes(int64_t BH, int64_t N) { return rot_offset_bytes(BH, N) + 2 * rot_bytes(BH, N); }

template <typename T, int MODE, bool DEV>
hipError_t run(const BwdArgs& a) {
  const int tiles = (int)tiles_of(a.N);
  const int64_t blocks = (int64_t)tiles * a.BH;
  const float scale = (float)(1.0 / sqrt((double)kD));
  float* delta = (float*)a.workspace;
  float* part = delta + ((a.BH * a.N + 63) / 64) * 64;
  dim3 grid((unsigned)blocks), block(256);
  int64_t n_part = blocks;
  uint32_t* ps = nullptr;  // per-(query, entry) P and dS, stored by the ring query side
  // interpolated: rotated query and key rows, written by the ring query side for the ring key
  // side
  bf16_t* qr = MODE == 1 ? (bf16_t*)((char*)a.workspace + rot_offset_bytes(a.BH, a.N)) : nullptr;
  bf16_t* kr = MODE == 1 ? qr + (size_t)a.BH * (size_t)a.N * kD : nullptr;
  const bool q_ring = bwdq_ring_supported(a);
  if (q_ring) {
    if (MODE == 1) ps = (uint32_t*)((char*)a.workspace + ps_offset_bytes(a.BH, a.N));
    const hipError_t e = launch_bwdq_ring(a, delta, part, ps, qr, kr);
    if (e != hipSuccess) return e;
    n_part = bwdq_ring_blocks(a);
  } else {
    bwd_query_kernel<T, MODE, DEV><<<grid, block, 0, a.stream>>>((const T*)a.q, (const T*)a.k, (const T*)a.v,
        (const T*)a.o, (const T*)a.dout, a.lse, (T*)a.dq, delta, part, a.N, a.W, a.tab, a.rope, scale, tiles,
        a.plan, a.heads_per_plan);
  }
  // the query-side workgroups are head-major, so each layer's partials are one run
  bool dalpha_done = false;
  if (bwdk_ring_supported(a) && (MODE == 0 || ps != nullptr)) {
    const hipError_t e = launch_bwdk_ring(a, delta, ps, part, n_part / a.layers, qr, kr);
    if (e != hipSuccess) return e;
    dalpha_done = true;  // the ring key side writes dalpha
  } else if (ps != nullptr) {
    bwd_key_ps_kernel<DEV><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
        (const bf16_t*)a.v, (const bf16_t*)a.dout, a.lse, delta, ps, (bf16_t*)a.dk, (bf16_t*)a.dv, a.N, a.W, a.tab,
        a.rope, scale, tiles, a.plan, a.heads_per_plan, a.ps_slots);
  } else {
    bwd_key_kernel<T, MODE, DEV><<<grid, block, 0, a.stream>>>((const T*)a.q, (const T*)a.k, (const T*)a.v,
        (const T*)a.dout, a.lse, delta, (T*)a.dk, (T*)a.dv, a.N, a.W, a.tab, a.rope, scale, tiles, a.plan, a.heads_per_plan);
  }
  if (a.dalpha != nullptr && !dalpha_done) {
    if (MODE == 1)
      dalpha_reduce_kernel<<<a.layers, 256, 0, a.stream>>>(part, n_part / a.layers, a.dalpha);
    else
      store_zero_kernel<<<1, 256, 0, a.stream>>>(a.dalpha, a.layers);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t BH, int64_t N, int dtype, int mode, int ps_slots) {
  if (dtype != 1 || mode != 1) return rot_offset_bytes(BH, N);
  return ps_offset_bytes(BH, N) + (size_t)BH * (size_t)ps_slots * (size_t)N * sizeof(uint32_t);
}

int ps_entry_slots(float alpha_hi, const int32_t* base, int n_base, int W) {
  // at least one slot: the ring key side reads (and discards) entry 0's words even when
  // the table is empty
  int n = 0;
  for (int e = 0; e < n_base; ++e)
    if ((double)alpha_hi * (double)base[e] >= (double)W) ++n;
  return n > 0 ? n : 1;
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.plan != nullptr) {
    if (a.dtype == 0) return a.mode == 0 ? run<float, 0, true>(a) : run<float, 1, true>(a);
    return a.mode == 0 ? run<bf16_t, 0, true>(a) : run<bf16_t, 1, true>(a);
  }
  if (a.dtype == 0) return a.mode == 0 ? run<float, 0, false>(a) : run<float, 1, false>(a);
  return a.mode == 0 ? run<bf16_t, 0, false>(a) : run<bf16_t, 1, false>(a);
}

}  // namespace fib
