// Single-query (decode) kernel of Fibonacci-offset dilated sparse attention: the newest
// position of a key/value cache attends its window and its offset keys.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science
// summaries of arXiv 2606.28560, Method > Architecture and attention mechanism; Results 2
// compares the inference cost of the integer and the interpolated gather): the query at
// position i = N - 1 attends the cache rows i, i-1, ..., i-W+1 and, per table entry, the row
// i - r (integer mode) or the blend (1-w) row(i-c) + w row(i-c+1) of K and V (interpolated
// mode), after RoPE; the result equals row N - 1 of the full forward over the cache.
//
// Design: one 256-thread block per (batch, head). The block's 64 lane quads take one key
// each (a window key or a table entry, "virtual" keys), all issued at once: a decode step is
// one round of memory latency, not a walk over the keys. Lane c of a quad owns dims
// 8c..8c+7 and 32+8c..32+8c+7 (8 complete RoPE pairs); RoPE is relative (only the query is
// rotated, by the key's distance, with cos/sin of the call's distances in LDS). Each quad
// keeps its own softmax state (more than 64 keys: several per quad, online); the block then
// merges the 64 states through LDS in a fixed order.
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

constexpr int kQuads = 64;

template <typename T, int MODE, bool DEV>
__global__ __launch_bounds__(256) void decode_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, T* __restrict__ o,
                                                     float* __restrict__ lse, int64_t N, int W, Table tab_arg,
                                                     Rope rope, float scale_log2, const DevPlan* __restrict__ plan,
                                                     int heads_per_plan) {
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)blockIdx.x / heads_per_plan);
  __shared__ float2 cs[kCsSlots][kHalf];
  __shared__ float red_m[kQuads], red_l[kQuads];
  __shared__ float red_o[kQuads][kD];
  const bool cached = fill_cs(cs, W, tab, MODE, rope);
  const int64_t head = blockIdx.x;
  const int c = threadIdx.x & 3;
  const int u = threadIdx.x >> 2;
  const int64_t i = N - 1;
  const T* kh_ = k + (size_t)head * (size_t)N * kD;
  const T* vh_ = v + (size_t)head * (size_t)N * kD;

  float ql[8], qh[8];
  Vec8<T>::load(q + (size_t)head * kD + 8 * c, ql);
  Vec8<T>::load(q + (size_t)head * kD + kHalf + 8 * c, qh);

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
  for (int64_t x = u; x < nv; x += kQuads) {
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

  // merge the states of the quads that took keys (quads 0..nv-1, all 64 when nv >= 64)
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
  if (threadIdx.x < kD) {
    const int dim = threadIdx.x;
    const int nq = nv < kQuads ? (int)nv : kQuads;  // quads that took a key
    float M = -INFINITY;
    for (int x = 0; x < nq; ++x) M = fmaxf(M, red_m[x]);  // finite: distance 0 always exists
    float L = 0.f, Od = 0.f;
    for (int x = 0; x < nq; ++x) {
      const float sc = exp2f(red_m[x] - M);
      L = fmaf(red_l[x], sc, L);
      Od = fmaf(red_o[x][dim], sc, Od);
    }
    const float val = Od / L;
    if constexpr (sizeof(T) == 4) {
      reinterpret_cast<float*>(o)[(size_t)head * kD + dim] = val;
    } else {
      reinterpret_cast<bf16_t*>(o)[(size_t)head * kD + dim] = (bf16_t)f2bf(val);
    }
    if (dim == 0 && lse != nullptr) lse[head] = (M + log2f(L)) * 0.69314718055994530942f;
  }
}

template <bool DEV>
hipError_t launch_decode_t(const FwdArgs& a) {
  dim3 grid((unsigned)a.BH), block(256);
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)kD));
  if (a.dtype == 0) {
    if (a.mode == 0)
      decode_kernel<float, 0, DEV><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
    else
      decode_kernel<float, 1, DEV><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
  } else {
    if (a.mode == 0)
      decode_kernel<bf16_t, 0, DEV><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
    else
      decode_kernel<bf16_t, 1, DEV><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, a.plan, a.heads_per_plan);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const FwdArgs& a) {
  return a.plan != nullptr ? launch_decode_t<true>(a) : launch_decode_t<false>(a);
}

}  // namespace fib
