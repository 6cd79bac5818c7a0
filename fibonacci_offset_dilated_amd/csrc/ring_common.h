// Device helpers shared by the LDS-ring kernels (forward and backward) of the
// Fibonacci-offset attention: ring geometry, MFMA and LDS-transpose wrappers, bf16 packing,
// RoPE rotation of a lane's 16 values, the per-query lane reductions and the diagonal
// P^T / dS^T block builder. See fwd_ring.hip for the layout these helpers assume: 16 queries
// (rows) per wave, lane (n, g) = (l & 15, l >> 4) holds row n, dims 8g..8g+7 and
// 32+8g..32+8g+7.
#pragma once

#include "fib_common.h"
#include "fib_launch.h"

#include <atomic>

namespace fib {
namespace ring {

// Raises a ring kernel's dynamic LDS limit to `bytes` on the current device, once per
// device and kernel instance (`done` holds one bit per device): the setting is idempotent,
// and repeating it on every launch costs host time that short calls notice.
template <typename K>
inline hipError_t ensure_lds_limit(K* kernel, std::atomic<uint32_t>& done, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = dev >= 0 && dev < 32 ? (1u << dev) : 0u;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) short s4;

constexpr int kP = 512;               // ring rows (a power of two: slot = row & (kP - 1))
constexpr int kRow = 144;             // ring row stride in bytes (128 + 16 padding)
// queries (and ring rows) per step: 16 per wave; the largest distance served from the ring
constexpr int step_rows(int waves) { return 16 * waves; }
constexpr int max_cov(int waves) { return kP - step_rows(waves); }
constexpr int kMaxBand = 16;          // window band rows before a 16-query block
constexpr int kMaxCov = 16;           // table entries served from the ring
constexpr int kMaxFar = 4;            // table entries served from global memory
constexpr int kMaxUnc = 2 * kMaxFar;  // their distances (interpolated: c and c - 1)
// Rows 0..kMirror-1 of the ring are also stored after its end, so that any 32 consecutive
// ring rows (slots s..s+31, s < kP) are one base address plus constant offsets.
constexpr int kMirror = 32;
static_assert(kP == kRingRows && kMaxBand == kBandRows && kMaxCov == kSplitCov && kMaxFar == kSplitFar,
              "ring geometry and RingSplit must agree");

// Queued table entries (forward): a distance a few steps beyond the ring reach whose 16-row
// slab is read from the ring `depth` steps before its queries run, while its rows are still
// there, and held in registers until then. The slab of the wave's queries p + 16w.. at
// distance d is rows p + 16w - d.. : read at step p - depth * T (T rows per step), they lie
// inside the ring then (ring rows p - depth T - reach .. p - depth T + T - 1) exactly when
// depth * T <= d <= reach + depth * T. Two queue slots, with these depths (interpolated
// mode uses the first).
constexpr int kMaxQ = 2;
constexpr int kQDepth0 = 2;
constexpr int kQDepth1 = 5;
constexpr bool queue_fits(int d, int depth, int waves) {
  return d > max_cov(waves) && depth * step_rows(waves) <= d && d <= max_cov(waves) + depth * step_rows(waves);
}
// Interpolated entries (distance c = ceil(alpha f)) read the 17 rows c back .. c - 16 back.
constexpr bool queue_fits_interp(int c, int depth, int waves) {
  return c > max_cov(waves) && depth * step_rows(waves) + 1 <= c && c <= max_cov(waves) + depth * step_rows(waves);
}

// byte offset of ring row `row` (any integer, negative rows included: slots are row mod kP);
// wave-uniform arguments keep it on the scalar unit
__device__ __forceinline__ int row_off(int row) { return (row & (kP - 1)) * kRow; }

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ uint32_t lds_read4(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint32_t*>(base + off);
}
__device__ __forceinline__ uint2 lds_read8(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint2*>(base + off);
}
__device__ __forceinline__ void lds_write16(uint8_t* base, int off, uint4 x) {
  *reinterpret_cast<uint4*>(base + off) = x;
}
__device__ __forceinline__ void lds_write8(uint8_t* base, int off, uint32_t x, uint32_t y) {
  *reinterpret_cast<uint2*>(base + off) = make_uint2(x, y);
}

// LDS transpose read of 4 bf16: lane j (of 16) supplies the address of 4 consecutive
// elements of row (k0 + j/4); lane i receives rows k0..k0+3 of column i.
__device__ __forceinline__ s4 tr16(const uint8_t* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(base + off));
}

__device__ __forceinline__ bf16x8 as_bf8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 cat_bf8(s4 a, s4 b) {
  typedef __attribute__((ext_vector_type(8))) short s8;
  s8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ f4 mfma32(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void unpack8(uint4 x, float* f) {
  f[0] = bf_lo(x.x); f[1] = bf_hi(x.x); f[2] = bf_lo(x.y); f[3] = bf_hi(x.y);
  f[4] = bf_lo(x.z); f[5] = bf_hi(x.z); f[6] = bf_lo(x.w); f[7] = bf_hi(x.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  uint4 x;
  x.x = pack_bf2(f[0], f[1]); x.y = pack_bf2(f[2], f[3]);
  x.z = pack_bf2(f[4], f[5]); x.w = pack_bf2(f[6], f[7]);
  return x;
}

// rotate the pairs (x[t], x[8 + t]) of 16 unpacked values by cos/sin cs[t]; packed bf16 halves
__device__ __forceinline__ void rotate_pack_f(const float* x, const float2* cs, uint4* out_lo, uint4* out_hi) {
  float ra[8], rb[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    ra[t] = x[t] * cs[t].x - x[8 + t] * cs[t].y;
    rb[t] = x[8 + t] * cs[t].x + x[t] * cs[t].y;
  }
  *out_lo = pack8(ra);
  *out_hi = pack8(rb);
}

// 2^x on the hardware unit (v_exp_f32); arguments here are <= 0 and results below the
// normal range are negligible softmax weights
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ bf16x2 as_bf2(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }
// c + x.lo * w.lo + x.hi * w.hi on bf16 pairs, fp32 accumulation (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2(uint32_t x, uint32_t w, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf2(x), as_bf2(w), c, false);
}

// select x[l & 3]
__device__ __forceinline__ float sel4(f4 x, int l) {
  const float a = (l & 1) ? x[1] : x[0];
  const float b = (l & 1) ? x[3] : x[2];
  return (l & 2) ? b : a;
}

// Reductions over the four lanes of a query (l, l ^ 16, l ^ 32, l ^ 48): each swap exchanges
// half of two copies of x, after which the pair holds x of both partner lanes.
__device__ __forceinline__ float quad_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const uint32_t w = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float quad_add(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const uint32_t w = __float_as_uint(x);
  auto s = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Diagonal P^T block of two slabs for the PV MFMA. The B operand of lane (n, g) holds slab-A
// rows 4g..4g+3 (slots 0-3) and slab-B rows 4g..4g+3 (slots 4-7) for query n; the diagonal
// weight of query n sits in lane g = n / 4, slot n % 4 (slab A) and 4 + n % 4 (slab B).
// x packs (weight A, weight B) as bf16 in the query's diagonal lane and zero elsewhere;
// sel[] are the lane's byte selectors (v_perm_b32) that place x's halves in those slots.
__device__ __forceinline__ bf16x8 diag_block(uint32_t x, const uint32_t* sel) {
  return __builtin_bit_cast(bf16x8, make_uint4(__builtin_amdgcn_perm(x, x, sel[0]), __builtin_amdgcn_perm(x, x, sel[1]),
                                               __builtin_amdgcn_perm(x, x, sel[2]), __builtin_amdgcn_perm(x, x, sel[3])));
}

// Element offset of the lane's row of a far entry's 16-row slab for the wave's queries
// i0w.. (row i0w - d + n; far distances exceed the ring reach, so the slab never passes row
// N - 1). lane_off = n * D + 8 g. A slab that starts before row 0 clamps each lane's row to
// row 0 (the queries that read rows before it are masked).
__device__ __forceinline__ int64_t far_off(int d, int i0w, int n, int g, int lane_off) {
  const int r0 = i0w - d;
  if (r0 >= 0) return (int64_t)r0 * kD + lane_off;
  return (int64_t)(r0 + n > 0 ? r0 + n : 0) * kD + 8 * g;
}

// Entries usable by some query (distance < N), split into the ring-covered prefix (distance
// <= the ring reach of a workgroup of `waves` waves) and the far rest (the table is sorted by
// distance in both modes).
inline void split_table(const Table& tab, int64_t N, int waves, int* n_cov, int* n_far) {
  int n = 0;
  while (n < tab.n && tab.dist[n] < N) ++n;
  const int cov_max = max_cov(waves);
  int cov = 0;
  while (cov < n && tab.dist[cov] <= cov_max) ++cov;
  *n_cov = cov;
  *n_far = n - cov;
}

// Segments per head for a launch of BH heads of `tiles` steps. Long sequences: about 512
// workgroups (two rounds over the 256 CUs; the second evens out the finishing times). When
// that would leave fewer than 8 steps per segment, each segment's warm-up (up to 3 steps of
// ring rows) weighs too much: one round of at most 256 workgroups instead.
inline int64_t ring_segments(int64_t BH, int64_t tiles) {
  int64_t segs = (512 + BH - 1) / BH;
  if ((tiles + segs - 1) / segs < 8) segs = 256 / BH;
  if (segs > tiles) segs = tiles;
  if (segs < 1) segs = 1;
  const int64_t per = (tiles + segs - 1) / segs;
  return (tiles + per - 1) / per;
}

// Interpolated far entry: the upper rows (i0w - d + 1 + n) from the lower rows (lane (n, g)
// holding row i0w - d + n, dims 8g.. and 32 + 8g..; ex: dword l % 32 of row i0w - d + 16).
// Lane n takes lane n + 1's row (DPP row shift within the 16 lanes of a dim group); lane 15
// takes row i0w - d + 16 from the dwords spread over the wave. Call with every lane of the
// wave active: both moves read other lanes' registers.
__device__ __forceinline__ void upper_rows(const uint4* lo, uint32_t ex, int g, uint4* hi) {
  uint32_t w[8] = {lo[0].x, lo[0].y, lo[0].z, lo[0].w, lo[1].x, lo[1].y, lo[1].z, lo[1].w};
  // (empty asm: the moves happen here, not hoisted to where their results would hold
  // registers through other work)
#pragma unroll
  for (int x = 0; x < 8; ++x) asm volatile("" : "+v"(w[x]));
  asm volatile("" : "+v"(ex));
  uint32_t h[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    // dword x of the lane's slice: 16-byte half x / 4 (dims 8g.. or 32 + 8g..), word x % 4
    const int src = 16 * (x >> 2) + 4 * g + (x & 3);
    const int e = __builtin_amdgcn_ds_bpermute(4 * src, (int)ex);
    h[x] = (uint32_t)__builtin_amdgcn_update_dpp(e, (int)w[x], 0x101, 0xf, 0xf, false);
  }
  hi[0] = make_uint4(h[0], h[1], h[2], h[3]);
  hi[1] = make_uint4(h[4], h[5], h[6], h[7]);
}

}  // namespace ring
}  // namespace fib
