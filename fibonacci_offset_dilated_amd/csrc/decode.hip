// Gather kernel of Fibonacci-offset dilated sparse attention: every key of a query requested
// at once. Serves the decode step (the newest position of a key/value cache attends its window
// and its offset keys) and the forward of small problems.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science
// summaries of arXiv 2606.28560, Method > Architecture and attention mechanism; Results 2
// compares the inference cost of the integer and the interpolated gather): the query at
// position i = N - 1 attends the cache rows i, i-1, ..., i-W+1 and, per table entry, the row
// i - r (integer mode) or the blend (1-w) row(i-c) + w row(i-c+1) of K and V (interpolated
// mode), after RoPE; the result equals row N - 1 of the full forward over the cache.
//
// Design: one 256-thread block per (batch, head) in decode, per 1, 2 or 4 consecutive queries of
// one head in the forward. The block's 64 lane quads (64 / QB per query) take one key each (a
// window key or a table entry, "virtual" keys), all issued at once: a query is one round of
// memory latency, not a walk over the keys. Lane c of a quad owns dims
// 8c..8c+7 and 32+8c..32+8c+7 (8 complete RoPE pairs); RoPE is relative (only the query is
// rotated, by the key's distance, with cos/sin of the call's distances in LDS). Each quad
// keeps its own softmax state (more than 64 keys: several per quad, online); the block then
// merges the 64 states through LDS in a fixed order.
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

constexpr int kQuads = 64;

// QB queries per block, 64 / QB lane quads per query. FWD: the block's queries are QB
// consecutive positions of one head (forward of small problems: every query's keys are
// requested at once instead of walked one after another); otherwise one query per (batch,
// head) at position N - 1 (decode).
template <typename T, int MODE, bool DEV, int QB, bool FWD>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, T* __restrict__ o,
                                                     float* __restrict__ lse, int64_t N, int W, Table tab_arg,
                                                     Rope rope, float scale_log2, const DevPlan* __restrict__ plan,
                                                     int heads_per_plan) {
  constexpr int kQpq = kQuads / QB;  // quads per query
  const int64_t bph = FWD ? (N + QB - 1) / QB : 1;  // blocks per head
  const int64_t head = FWD ? (int64_t)blockIdx.x / bph : (int64_t)blockIdx.x;
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)(head / heads_per_plan));
  __shared__ float2 cs[kCsSlots][kHalf];
  __shared__ float red_m[kQuads], red_l[kQuads];
  __shared__ float red_o[kQuads][kD];
  const bool cached = fill_cs(cs, W, tab, MODE, rope);
  const int c = threadIdx.x & 3;
  const int u = threadIdx.x >> 2;
  const int qb = u / kQpq;  // the quad's query within the block
  const int uq = u % kQpq;  // the quad within its query
  const int64_t i_raw = FWD ? ((int64_t)blockIdx.x % bph) * QB + qb : N - 1;
  const bool valid = i_raw < N;
  const int64_t i = valid ? i_raw : N - 1;  // (a query past the end repeats the last: not stored)
  const T* kh_ = k + (size_t)head * (size_t)N * kD;
  const T* vh_ = v + (size_t)head * (size_t)N * kD;
  const T* qrow = q + (FWD ? ((size_t)head * (size_t)N + (size_t)i) : (size_t)head) * kD;

  float ql[8], qh[8];
  Vec8<T>::load(qrow + 8 * c, ql);
  Vec8<T>::load(qrow + kHalf + 8 * c, qh);

  // virtual keys: window distances 0..wv-1, then the entries usable at i (a prefix: the
  // table is sorted by distance)
  const int64_t wv = (int64_t)W < i + 1 ? (int64_t)W : i + 1;
  int ne = 0;
  while (ne < tab.n && (int64_t)tab.dist[ne] <= i) ++ne;
  const int64_t nv = wv + ne;

  float acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.f;
  float m = -INFINITY, l = 0.f;
  float kl[8], kh[8], vl[8], vh[8], rl[8], rh[8];
  for (int64_t x = uq; x < nv; x += kQpq) {
    float s;
    if (x < wv) {
      const int64_t j = i - x;
      Vec8<T>::load(kh_ + j * kD + 8 * c, kl);
      Vec8<T>::load(kh_ + j * kD + kHalf + 8 * c, kh);
      Vec8<T>::load(vh_ + j * kD + 8 * c, vl);
      Vec8<T>::load(vh_ + j * kD + kHalf + 8 * c, vh);
      rotate8(ql, qh, rl, rh, cs, cached, (int)x, x, c, rope);
      s = dot16(rl, rh, kl, kh);
    } else {
      const int e = (int)(x - wv);
      const int64_t d = tab.dist[e];
      const int64_t lo = i - d;
      Vec8<T>::load(kh_ + lo * kD + 8 * c, kl);
      Vec8<T>::load(kh_ + lo * kD + kHalf + 8 * c, kh);
      Vec8<T>::load(vh_ + lo * kD + 8 * c, vl);
      Vec8<T>::load(vh_ + lo * kD + kHalf + 8 * c, vh);
      rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
      s = dot16(rl, rh, kl, kh);
      if (MODE == 1) {
        // virtual key (1-w) row(lo) + w row(lo+1), the same blend of V rows
        const float w = tab.w[e];
        float kl2[8], kh2[8], vl2[8], vh2[8];
        Vec8<T>::load(kh_ + (lo + 1) * kD + 8 * c, kl2);
        Vec8<T>::load(kh_ + (lo + 1) * kD + kHalf + 8 * c, kh2);
        Vec8<T>::load(vh_ + (lo + 1) * kD + 8 * c, vl2);
        Vec8<T>::load(vh_ + (lo + 1) * kD + kHalf + 8 * c, vh2);
        rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
        s = fmaf(w, dot16(rl, rh, kl2, kh2) - s, s);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          vl[t] = fmaf(w, vl2[t] - vl[t], vl[t]);
          vh[t] = fmaf(w, vh2[t] - vh[t], vh[t]);
        }
      }
    }
    // online softmax of the quad's keys, base-2 logits
    s = quad_sum(s) * scale_log2;
    const float mn = fmaxf(m, s);
    const float corr = exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = fmaf(l, corr, p);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] = fmaf(acc[t], corr, p * vl[t]);
      acc[8 + t] = fmaf(acc[8 + t], corr, p * vh[t]);
    }
    m = mn;
  }

  // merge, per query, the states of its quads that took keys (all kQpq when nv >= kQpq)
  if (c == 0) {
    red_m[u] = m;
    red_l[u] = l;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    red_o[u][8 * c + t] = acc[t];
    red_o[u][kHalf + 8 * c + t] = acc[8 + t];
  }
  __syncthreads();
  if (threadIdx.x < QB * kD) {
    const int qq = threadIdx.x / kD;  // query slot: its quads are qq * kQpq ...
    const int dim = threadIdx.x % kD;
    const int64_t iq_raw = FWD ? ((int64_t)blockIdx.x % bph) * QB + qq : N - 1;
    const int64_t iq = iq_raw < N ? iq_raw : N - 1;
    const int64_t wq = (int64_t)W < iq + 1 ? (int64_t)W : iq + 1;
    int neq = 0;
    while (neq < tab.n && (int64_t)tab.dist[neq] <= iq) ++neq;
    const int64_t nvq = wq + neq;
    const int nq = nvq < kQpq ? (int)nvq : kQpq;  // quads that took a key
    const int u0 = qq * kQpq;
    float M = -INFINITY;
    for (int x = 0; x < nq; ++x) M = fmaxf(M, red_m[u0 + x]);  // finite: distance 0 always exists
    float L = 0.f, Od = 0.f;
    for (int x = 0; x < nq; ++x) {
      const float sc = exp2f(red_m[u0 + x] - M);
      L = fmaf(red_l[u0 + x], sc, L);
      Od = fmaf(red_o[u0 + x][dim], sc, Od);
    }
    const float val = Od / L;
    const size_t orow = FWD ? (size_t)head * (size_t)N + (size_t)iq : (size_t)head;
    if (iq_raw < N) {
      if constexpr (sizeof(T) == 4) {
        reinterpret_cast<float*>(o)[orow * kD + dim] = val;
      } else {
        reinterpret_cast<bf16_t*>(o)[orow * kD + dim] = (bf16_t)f2bf(val);
      }
      if (dim == 0 && lse != nullptr) lse[orow] = (M + log2f(L)) * 0.69314718055994530942f;
    }
  }
}

template <bool DEV, int QB, bool FWD>
hipError_t launch_gather_t(const FwdArgs& a) {
  const int64_t blocks = FWD ? a.BH * ((a.N + QB - 1) / QB) : a.BH;
  dim3 grid((unsigned)blocks), block(256);
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)kD));
  if (a.dtype == 0) {
    if (a.mode == 0)
      gather_kernel<float, 0, DEV, QB, FWD><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
    else
      gather_kernel<float, 1, DEV, QB, FWD><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
  } else {
    if (a.mode == 0)
      gather_kernel<bf16_t, 0, DEV, QB, FWD><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
    else
      gather_kernel<bf16_t, 1, DEV, QB, FWD><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
  }
  return hipGetLastError();
}

// largest virtual-key count of the call (window plus table entries; with alpha in device
// memory, every base entry may be kept)
int max_virtual_keys(const FwdArgs& a) {
  const int n = a.plan != nullptr ? a.n_base : a.tab.n;
  return a.W + n;
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a) {
  return a.plan != nullptr ? launch_gather_t<true, 1, false>(a) : launch_gather_t<false, 1, false>(a);
}

bool fwd_gather_preferred(const FwdArgs& a) {
  // small problems, where walking a query's keys one after another leaves the call
  // latency-bound; larger ones amortise the block's cos/sin table over 64 queries in the
  // general kernel
  return a.BH * a.N <= kGatherMaxRows;
}

hipError_t launch_fwd_gather(const FwdArgs& a) {
  // queries per block: as many as leave 64 / QB quads >= the virtual keys of a query
  const int nv = max_virtual_keys(a);
  const int qb = nv <= 16 ? 4 : nv <= 32 ? 2 : 1;
  if (a.plan != nullptr) {
    if (qb == 4) return launch_gather_t<true, 4, true>(a);
    if (qb == 2) return launch_gather_t<true, 2, true>(a);
    return launch_gather_t<true, 1, true>(a);
  }
  if (qb == 4) return launch_gather_t<false, 4, true>(a);
  if (qb == 2) return launch_gather_t<false, 2, true>(a);
  return launch_gather_t<false, 1, true>(a);
}

}  // namespace fib
