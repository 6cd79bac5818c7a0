// Device-side types and helpers shared by the Fibonacci-offset attention kernels (gfx950).
//
// The operation is the attention layer of "Depth-Staggered Fibonacci Spacing for Sparse
// Attention" (gist.science summaries of arXiv 2606.28560), Method > Architecture and
// attention mechanism: window of W keys plus offsets d_k = alpha * f_k, interpolated K/V
// rows for non-integer d_k, RoPE before the gather.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace fib {

constexpr int kD = 64;        // head size supported by the kernels
constexpr int kHalf = kD / 2; // RoPE pairs (j, j + D/2)
constexpr int kMaxEnt = 32;   // offset-table capacity (= max base length)

typedef uint16_t bf16_t;      // bf16 stored as raw bits

// Offset table of one call: integer mode keeps sorted offsets r in dist[]; interpolated mode
// keeps ceil(alpha f) in dist[], the weight of the upper row in w[] and f in f[].
struct Table {
  int n;
  int dist[kMaxEnt];
  float w[kMaxEnt];
  float f[kMaxEnt];
};

// Offset table of one call ("Depth-Staggered Fibonacci Spacing for Sparse Attention", Method >
// Architecture and attention mechanism: d = alpha f per base offset f). mode 0 (integer):
// r = round-half-to-even(alpha f), kept when r >= W, equal offsets collapse; mode 1
// (interpolated): kept when alpha f >= W, c = ceil(alpha f), w = c - alpha f. alpha * f is
// exact in fp64 (a 24-bit significand times f <= 2^24), so the rounding (rint: ties to even
// in the default rounding mode) and the ceiling act on the true product. The same code
// builds the table on the host and, for an alpha held in device memory, on the device.
__host__ __device__ inline void build_table(float alpha, const int32_t* base, int n_base, int W, int mode,
                                            Table* t) {
  t->n = 0;
  for (int e = 0; e < kMaxEnt; ++e) {
    t->dist[e] = 0;
    t->w[e] = 0.f;
    t->f[e] = 0.f;
  }
  for (int e = 0; e < n_base; ++e) {
    const double d = (double)alpha * (double)base[e];
    if (mode == 0) {
      const double r = rint(d);
      if (r < (double)W || r > 2147483647.0) continue;
      if (t->n > 0 && t->dist[t->n - 1] == (int)r) continue;  // r is non-decreasing in f
      t->dist[t->n] = (int)r;
      t->n++;
    } else {
      if (d < (double)W) continue;
      const double c = ceil(d);
      if (c > 2147483647.0) continue;
      t->dist[t->n] = (int)c;
      t->w[t->n] = (float)(c - d);
      t->f[t->n] = (float)base[e];
      t->n++;
    }
  }
}

// The table of a call: the kernel argument, or (DEV instances, alpha in device memory) the
// one built on the device for the block's layer. The pointer is a read-only kernel argument
// and the layer is uniform, so its loads are uniform (scalar) loads.
template <bool DEV, typename Plan>
__device__ __forceinline__ const Table& call_table(const Table& arg, const Plan* plan, int layer) {
  if constexpr (DEV) return plan[layer].tab;
  else return arg;
}

// RoPE rates in revolutions per position: omega_j / (2 pi), omega_j = theta^(-2j/D), fp64.
struct Rope {
  double rev[kHalf];
};

// cos and sin of the RoPE angle p * omega_j. The angle is reduced in fp64 (p * rev, minus
// the nearest integer number of turns) before the fp32 sincos, so it stays accurate for
// positions far beyond fp32's integer range of exact angles.
__device__ __forceinline__ float2 rope_cs(int64_t p, double rev) {
  double t = (double)p * rev;
  t -= rint(t);
  float a = (float)(t * 6.283185307179586476925286766559);
  float s, c;
  sincosf(a, &s, &c);
  return make_float2(c, s);
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN stays NaN): the hardware conversion
// v_cvt_pk_bf16_f32, two values per instruction.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f2bf(float x) { return pack_bf2(x, 0.f) & 0xffffu; }

// (P, dS) of one (query, table entry) in 32 bits, handed from the query side of the
// interpolated backward to its key side: dS as an fp32 whose mantissa is rounded (to
// nearest even) to 11 bits (bits 31..12: 12 significant bits, against bf16's 8), P in [0, 1]
// as a 12-bit fixed-point fraction P * 4095 (bits 11..0; absolute error <= 1.3e-4).
__device__ __forceinline__ uint32_t ps_pack(float p, float ds) {
  uint32_t u = __float_as_uint(ds);
  u = (u + 0x7ffu + ((u >> 12) & 1u)) & 0xfffff000u;
  const uint32_t q = (uint32_t)__builtin_rintf(fminf(fmaxf(p, 0.f), 1.f) * 4095.f);
  return u | q;
}
__device__ __forceinline__ float ps_ds(uint32_t x) { return __uint_as_float(x & 0xfffff000u); }
__device__ __forceinline__ float ps_p(uint32_t x) { return (float)(x & 0xfffu) * (1.f / 4095.f); }

// 8 consecutive elements <-> 8 floats
template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
};
template <> struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* x) {
    uint4 a = *reinterpret_cast<const uint4*>(p);
    x[0] = bf_lo(a.x); x[1] = bf_hi(a.x); x[2] = bf_lo(a.y); x[3] = bf_hi(a.y);
    x[4] = bf_lo(a.z); x[5] = bf_hi(a.z); x[6] = bf_lo(a.w); x[7] = bf_hi(a.w);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* x) {
    uint4 a;
    a.x = pack_bf2(x[0], x[1]); a.y = pack_bf2(x[2], x[3]);
    a.z = pack_bf2(x[4], x[5]); a.w = pack_bf2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = a;
  }
};

// Attended rows of query i for table entry e: the lower row (or the only row) and whether
// the entry is valid for i. Integer mode: row i - r_e, valid when r_e <= i. Interpolated
// mode: rows i - c_e and i - c_e + 1, valid when c_e <= i.
__device__ __forceinline__ bool entry_row(const Table& t, int e, int64_t i, int64_t* lo) {
  int64_t d = t.dist[e];
  *lo = i - d;
  return d <= i;
}

// ---- cos/sin of the RoPE angles at the few distances a call uses -----------------------
// Relative RoPE: <R_i q, R_j k> = <R_(i-j) q, k>, so the general kernels rotate only the
// query, by the key's distance. The distances are the window distances s < W, the table
// distances dist[e] and (interpolated mode) dist[e] - 1. Slot map: s -> s, entry e ->
// W + e, upper row of entry e -> W + n + e. When W + 2n <= kCsSlots the block fills an
// LDS table once; otherwise the angles are computed at each use.
constexpr int kCsSlots = 128;

__device__ __forceinline__ int64_t slot_dist(int slot, int W, const Table& t) {
  if (slot < W) return slot;
  if (slot < W + t.n) return t.dist[slot - W];
  return (int64_t)t.dist[slot - W - t.n] - 1;
}

// Fills cs[slot][j] for every slot when they fit; returns whether they did. Contains a
// block-wide barrier, so every thread of the block must call it.
__device__ __forceinline__ bool fill_cs(float2 (*cs)[kHalf], int W, const Table& t, int mode, const Rope& rope) {
  const bool fits = W <= kCsSlots && W + t.n * (mode == 1 ? 2 : 1) <= kCsSlots;
  const int slots = fits ? W + t.n * (mode == 1 ? 2 : 1) : 0;
  if (fits) {
    for (int idx = threadIdx.x; idx < slots * kHalf; idx += blockDim.x) {
      const int slot = idx / kHalf, j = idx % kHalf;
      cs[slot][j] = rope_cs(slot_dist(slot, W, t), rope.rev[j]);
    }
  }
  __syncthreads();
  return fits;
}

// Lane-quad helpers: lane c of a quad holds dims 8c..8c+7 (lo) and 32+8c..32+8c+7 (hi),
// i.e. the RoPE pairs j = 8c + t, t < 8.
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

__device__ __forceinline__ float2 get_cs(const float2 (*cs)[kHalf], bool cached, int slot, int64_t dist, int j,
                                         const Rope& rope) {
  return cached ? cs[slot][j] : rope_cs(dist, rope.rev[j]);
}


// r = R_dist x (rotation by +dist * omega_j) of the lane's 8 pairs.
__device__ __forceinline__ void rotate8(const float* xl, const float* xh, float* rl, float* rh,
                                        const float2 (*cs)[kHalf], bool cached, int slot, int64_t dist,
                                        int c, const Rope& rope) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float2 a = get_cs(cs, cached, slot, dist, 8 * c + t, rope);
    rl[t] = xl[t] * a.x - xh[t] * a.y;
    rh[t] = xh[t] * a.x + xl[t] * a.y;
  }
}

__device__ __forceinline__ float dot16(const float* al, const float* ah, const float* bl, const float* bh) {
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    s = fmaf(al[t], bl[t], s);
    s = fmaf(ah[t], bh[t], s);
  }
  return s;
}

}  // namespace fib
