// General forward kernel of Fibonacci-offset dilated sparse attention (any W, fp32 or bf16,
// integer or interpolated offsets). The bf16 workloads with W <= 16 run on the ring kernel
// (fwd_ring.hip); this kernel covers every other argument combination.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science
// summaries, Method > Architecture and attention mechanism): query i attends the window
// rows i, i-1, ..., i-W+1 and, per table entry, the row i - r (integer mode) or the blend
// (1-w) row(i-c) + w row(i-c+1) of K and V (interpolated mode); RoPE is applied to Q and K
// before the gather.
//
// Layout: 4 lanes per query ("quad"); lane c of a quad owns dims 8c..8c+7 and 32+8c..32+8c+7,
// i.e. 8 complete RoPE pairs. A 256-thread block handles 64 consecutive queries of one head.
// RoPE is applied in relative form: <R_i q, R_j k> = <R_(i-j) q, k>, so only the query is
// rotated, by the key's distance; K and V are read un-rotated. Softmax is online in fp32.
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

constexpr int kQPB = 64;  // queries per block

template <typename T, int MODE, bool DEV>
__global__ __launch_bounds__(256) void fwd_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* __restrict__ o,
    float* __restrict__ lse, int64_t N, int W, Table tab_arg, Rope rope, float scale_log2, int tiles,
    const DevPlan* __restrict__ plan, int heads_per_plan) {
  const Table& tab = call_table<DEV>(tab_arg, plan, (int)(blockIdx.x / tiles) / heads_per_plan);
  __shared__ float2 cs[kCsSlots][kHalf];
  const bool cached = fill_cs(cs, W, tab, MODE, rope);
  const int64_t head = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  const int c = threadIdx.x & 3;
  const int64_t i = (int64_t)tile * kQPB + (threadIdx.x >> 2);
  const bool active = i < N;
  const int64_t ii = active ? i : N - 1;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const T* qh_ = q + hoff;
  const T* kh_ = k + hoff;
  const T* vh_ = v + hoff;

  float ql[8], qh[8];
  Vec8<T>::load(qh_ + ii * kD + 8 * c, ql);
  Vec8<T>::load(qh_ + ii * kD + kHalf + 8 * c, qh);

  float acc[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) acc[t] = 0.f;
  float m = -INFINITY, l = 0.f;

  // online softmax over base-2 logits; s is the lane's partial dot product
  auto update = [&](float s, const float* vl, const float* vh) {
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
    update(dot16(rl, rh, kl, kh), vl, vh);
  }
  for (int e = 0; e < tab.n; ++e) {
    int64_t lo;
    if (!entry_row(tab, e, ii, &lo)) continue;
    Vec8<T>::load(kh_ + lo * kD + 8 * c, kl);
    Vec8<T>::load(kh_ + lo * kD + kHalf + 8 * c, kh);
    Vec8<T>::load(vh_ + lo * kD + 8 * c, vl);
    Vec8<T>::load(vh_ + lo * kD + kHalf + 8 * c, vh);
    const int64_t d = tab.dist[e];
    rotate8(ql, qh, rl, rh, cs, cached, W + e, d, c, rope);
    if (MODE == 0) {
      update(dot16(rl, rh, kl, kh), vl, vh);
    } else {
      // virtual key (1-w) row(lo) + w row(lo+1); lo + 1 <= i whenever lo is valid
      const float w = tab.w[e];
      float s = (1.f - w) * dot16(rl, rh, kl, kh);
      Vec8<T>::load(kh_ + (lo + 1) * kD + 8 * c, kl);
      Vec8<T>::load(kh_ + (lo + 1) * kD + kHalf + 8 * c, kh);
      rotate8(ql, qh, rl, rh, cs, cached, W + tab.n + e, d - 1, c, rope);
      s = fmaf(w, dot16(rl, rh, kl, kh), s);
      float vl2[8], vh2[8];
      Vec8<T>::load(vh_ + (lo + 1) * kD + 8 * c, vl2);
      Vec8<T>::load(vh_ + (lo + 1) * kD + kHalf + 8 * c, vh2);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        vl[t] = fmaf(w, vl2[t] - vl[t], vl[t]);
        vh[t] = fmaf(w, vh2[t] - vh[t], vh[t]);
      }
      update(s, vl, vh);
    }
  }
  if (!active) return;
  const float inv = 1.f / l;
  float outl[8], outh[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    outl[t] = acc[t] * inv;
    outh[t] = acc[8 + t] * inv;
  }
  T* oh = o + hoff;
  Vec8<T>::store(oh + i * kD + 8 * c, outl);
  Vec8<T>::store(oh + i * kD + kHalf + 8 * c, outh);
  if (lse != nullptr && c == 0) lse[(size_t)head * N + i] = (m + log2f(l)) * 0.69314718055994530942f;
}

template <bool DEV>
hipError_t launch_generic(const FwdArgs& a) {
  const int tiles = (int)((a.N + kQPB - 1) / kQPB);
  dim3 grid((unsigned)(tiles * a.BH)), block(256);
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)kD));
  if (a.dtype == 0) {
    if (a.mode == 0)
      fwd_generic_kernel<float, 0, DEV><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, tiles, a.plan, a.heads_per_plan);
    else
      fwd_generic_kernel<float, 1, DEV><<<grid, block, 0, a.stream>>>((const float*)a.q, (const float*)a.k,
          (const float*)a.v, (float*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, tiles, a.plan, a.heads_per_plan);
  } else {
    if (a.mode == 0)
      fwd_generic_kernel<bf16_t, 0, DEV><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, tiles, a.plan, a.heads_per_plan);
    else
      fwd_generic_kernel<bf16_t, 1, DEV><<<grid, block, 0, a.stream>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
          (const bf16_t*)a.v, (bf16_t*)a.o, a.lse, a.N, a.W, a.tab, a.rope, sl2, tiles, a.plan, a.heads_per_plan);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_generic(const FwdArgs& a) {
  return a.plan != nullptr ? launch_generic<true>(a) : launch_generic<false>(a);
}

// Debug export of the attended rows (same table and validity code as the kernels).
namespace {
__global__ void index_set_kernel(int32_t* out, int64_t N, int W, Table tab, int64_t cols) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  int32_t* row = out + i * cols;
  for (int s = 0; s < W; ++s) row[s] = (int64_t)s <= i ? (int32_t)(i - s) : -1;
  for (int e = 0; e < tab.n; ++e) {
    int64_t lo;
    row[W + e] = entry_row(tab, e, i, &lo) ? (int32_t)lo : -1;
  }
}
}  // namespace

hipError_t launch_index_set(int32_t* out, int64_t N, int W, const Table& tab, int64_t cols, hipStream_t s) {
  dim3 grid((unsigned)((N + 255) / 256)), block(256);
  index_set_kernel<<<grid, block, 0, s>>>(out, N, W, tab, cols);
  return hipGetLastError();
}

}  // namespace fib
