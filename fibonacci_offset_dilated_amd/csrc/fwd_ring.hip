// Fast forward kernel of Fibonacci-offset dilated sparse attention: bf16, D = 64, W <= 16,
// integer and interpolated offsets.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science summaries
// of arXiv 2606.28560, Method > Architecture and attention mechanism): query i attends the
// window rows i-W+1..i and one (integer mode) or one interpolated pair of (interpolated mode)
// rows per table entry, after RoPE; Results 2 notes that static offsets allow a fused path,
// which this kernel is for both modes.
//
// Design (gfx950):
//  * One 256-thread workgroup (4 waves) per CU sweeps a contiguous segment of one head in
//    steps of 64 queries; wave w owns queries p0 + 16w .. p0 + 16w + 15 of each step.
//  * LDS ring of the last kP rows: K rotated by RoPE (bf16) and raw V (bf16). Each row is
//    loaded from HBM and rotated once, when it enters the ring; the window band and every
//    table entry whose distance is <= kP - 64 read it from LDS afterwards.
//  * Logits on MFMA as S^T = K^ Q^T (v_mfma_f32_16x16x32_bf16; A = 16 key rows from the ring,
//    B = the wave's 16 rotated queries). The window band is a 32-key by 16-query block; a
//    table entry is a 16-row slab whose diagonal holds the 16 logits (query n reads slab
//    row n), picked out of the lanes that own it.
//  * Table entries beyond the ring read raw K rows from global memory and use relative RoPE:
//    <R_i q, R_(i-d) k> = <R_d q, k>, with cos/sin of R_d computed once per workgroup.
//  * Softmax over all logits of a query at once (they fit in registers), fp32, base 2.
//  * P V on MFMA as O^T = V^T P^T: V^T operands come from the ring through the LDS transpose
//    read (ds_read_b64_tr_b16); table entries use a diagonal P^T block, two slabs per MFMA
//    (interpolated mode: the lower and upper slab of one entry, weights 1-w and w).
//  * Ring rows use a 16-byte-chunk XOR swizzle (chunk ^ (slot & 7)) against bank conflicts.
#include "fib_common.h"
#include "fib_launch.h"

namespace fib {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) short s4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 16 * kWaves;       // queries (and ring rows) per step
constexpr int kP = 576;               // ring rows
constexpr int kMaxCov = kP - kT;      // largest distance served from the ring
constexpr int kMaxBand = 16;          // window band rows before a 16-query block
constexpr int kMaxUnc = 8;            // distances served from global memory
constexpr int kStageRows = 17;        // per-wave staging rows for V of far entries

struct RingArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  int64_t N;
  int W;
  int n_ent;        // table entries
  int n_cov;        // entries served from the ring (a prefix of the table)
  int n_unc;        // far distances (integer: one per far entry; interpolated: c and c-1)
  int seg_len;      // rows per workgroup (multiple of kT)
  int segs;         // segments per head
  int warm;         // rows inserted before the segment start (multiple of kT)
  float scale_log2;
  int dist[kMaxEnt];
  float w[kMaxEnt];
  int unc_dist[kMaxUnc];
  Rope rope;
};

struct __align__(16) Smem {
  uint8_t ringK[kP * 128];
  uint8_t ringV[kP * 128];
  uint8_t stage[kWaves][kStageRows * 128];
  float2 unc_cs[kMaxUnc][kHalf];
  float2 base_cs[2][kHalf];
};

__device__ __forceinline__ int slot_of(int64_t row) {
  // rows may be negative by up to kP (zero-filled ring slots stand for them)
  return (int)((row + (int64_t)kP * 4) % kP);
}
__device__ __forceinline__ int chunk_off(int slot, int chunk) { return slot * 128 + ((chunk ^ (slot & 7)) << 4); }

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, int off) {
  return *reinterpret_cast<const uint4*>(base + off);
}
__device__ __forceinline__ void lds_write16(uint8_t* base, int off, uint4 x) {
  *reinterpret_cast<uint4*>(base + off) = x;
}

// LDS transpose read of 4 bf16: lane j (of 16) supplies the address of 4 consecutive
// elements of row (k0 + j/4); lane i receives rows k0..k0+3 of column i.
__device__ __forceinline__ s4 tr16(const uint8_t* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(base + off));
}

__device__ __forceinline__ bf16x8 as_bf8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 cat_bf8(s4 a, s4 b) {
  typedef __attribute__((ext_vector_type(8))) short s8;
  s8 c = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, c);
}
__device__ __forceinline__ bf16x4 as_bf4(s4 a) { return __builtin_bit_cast(bf16x4, a); }

__device__ __forceinline__ f4 mfma32(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(bf16x4 a, bf16x4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
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

// rotate pairs (lo[t], hi[t]) by angles with cos/sin cs[t]; returns packed bf16 halves
__device__ __forceinline__ void rotate_pack(uint4 lo, uint4 hi, const float2* cs, uint4* out_lo, uint4* out_hi) {
  float a[8], b[8], ra[8], rb[8];
  unpack8(lo, a);
  unpack8(hi, b);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    ra[t] = a[t] * cs[t].x - b[t] * cs[t].y;
    rb[t] = b[t] * cs[t].x + a[t] * cs[t].y;
  }
  *out_lo = pack8(ra);
  *out_hi = pack8(rb);
}

// value of x rounded to bf16 (nearest even), as fp32
__device__ __forceinline__ float round_bf(float x) { return __uint_as_float(f2bf(x) << 16); }

// select x[l & 3]
__device__ __forceinline__ float sel4(f4 x, int l) {
  float a = (l & 1) ? x[1] : x[0];
  float b = (l & 1) ? x[3] : x[2];
  return (l & 2) ? b : a;
}

// 4 bf16 slots with value p at slot (l & 3), zeros elsewhere (as 2 packed dwords)
__device__ __forceinline__ void diag_slots(float p, int l, bool diag, uint32_t* d0, uint32_t* d1) {
  const uint32_t b = diag ? f2bf(p) : 0u;
  const int s = l & 3;
  *d0 = s == 0 ? b : (s == 1 ? (b << 16) : 0u);
  *d1 = s == 2 ? b : (s == 3 ? (b << 16) : 0u);
}

__device__ __forceinline__ float wave_xor_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_xor_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void fwd_ring_kernel(RingArgs a) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int n = l & 15;   // query (and row) within the wave's 16
  const int g = l >> 4;   // lane group: dims 8g..8g+7 and 32+8g..32+8g+7
  const bool diag_lane = g == (n >> 2);

  const int64_t head = blockIdx.x / a.segs;
  const int seg = blockIdx.x % a.segs;
  const int64_t N = a.N;
  const int64_t s0 = (int64_t)seg * a.seg_len;
  const int64_t s1 = s0 + a.seg_len < N ? s0 + a.seg_len : N;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const bf16_t* Qh = a.q + hoff;
  const bf16_t* Kh = a.k + hoff;
  const bf16_t* Vh = a.v + hoff;

  // ---- set-up: zero the ring, cos/sin of the far distances and of the first step base
  {
    uint4* z = reinterpret_cast<uint4*>(sm.ringK);
    const int n16 = (2 * kP * 128) / 16;
    for (int x = tid; x < n16; x += kThreads) z[x] = make_uint4(0, 0, 0, 0);
    for (int x = tid; x < a.n_unc * kHalf; x += kThreads) {
      const int u = x / kHalf, j = x % kHalf;
      sm.unc_cs[u][j] = rope_cs(a.unc_dist[u], a.rope.rev[j]);
    }
  }
  int64_t p0 = s0 - a.warm;
  if (p0 < 0) p0 = 0;
  if (tid < kHalf) sm.base_cs[0][tid] = rope_cs(p0, a.rope.rev[tid]);
  // per-lane rotation by t = 16 wave + n (the row's offset from the step base)
  float2 cs_t[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) cs_t[t] = rope_cs(16 * wave + n, a.rope.rev[8 * g + t]);
  __syncthreads();

  // prefetch of the rows this lane inserts: q/k/v dims 8g.. and 32+8g.. of row p0 + 16w + n
  auto load_rows = [&](int64_t pb, uint4* q2, uint4* k2, uint4* v2) {
    const int64_t r = pb + 16 * wave + n;
    if (r < N) {
      const bf16_t* qp = Qh + r * kD;
      const bf16_t* kp = Kh + r * kD;
      const bf16_t* vp = Vh + r * kD;
      q2[0] = *reinterpret_cast<const uint4*>(qp + 8 * g);
      q2[1] = *reinterpret_cast<const uint4*>(qp + kHalf + 8 * g);
      k2[0] = *reinterpret_cast<const uint4*>(kp + 8 * g);
      k2[1] = *reinterpret_cast<const uint4*>(kp + kHalf + 8 * g);
      v2[0] = *reinterpret_cast<const uint4*>(vp + 8 * g);
      v2[1] = *reinterpret_cast<const uint4*>(vp + kHalf + 8 * g);
    } else {
      q2[0] = q2[1] = k2[0] = k2[1] = v2[0] = v2[1] = make_uint4(0, 0, 0, 0);
    }
  };
  uint4 pq[2], pk[2], pv[2];
  load_rows(p0, pq, pk, pv);

  const float sl2 = a.scale_log2;
  int buf = 0;
  for (; p0 < s1; p0 += kT, buf ^= 1) {
    // ---- insert rows p0 + 16w + n: rotate K (and Q for this step's queries) by R_(p0 + t)
    float2 cs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 b = sm.base_cs[buf][8 * g + t];
      cs[t] = make_float2(b.x * cs_t[t].x - b.y * cs_t[t].y, b.y * cs_t[t].x + b.x * cs_t[t].y);
    }
    uint4 kr0, kr1, qh0, qh1;
    rotate_pack(pk[0], pk[1], cs, &kr0, &kr1);
    rotate_pack(pq[0], pq[1], cs, &qh0, &qh1);
    const uint4 qraw0 = pq[0], qraw1 = pq[1];
    {
      const int sl = slot_of(p0 + 16 * wave + n);
      lds_write16(sm.ringK, chunk_off(sl, g), kr0);
      lds_write16(sm.ringK, chunk_off(sl, 4 + g), kr1);
      lds_write16(sm.ringV, chunk_off(sl, g), pv[0]);
      lds_write16(sm.ringV, chunk_off(sl, 4 + g), pv[1]);
    }
    __syncthreads();
    // next step's rows and base rotation
    const int64_t pn = p0 + kT;
    if (pn < s1) load_rows(pn, pq, pk, pv);
    if (wave == 0 && l < kHalf) sm.base_cs[buf ^ 1][l] = rope_cs(pn, a.rope.rev[l]);

    if (p0 >= s0) {
      const int64_t i0w = p0 + 16 * wave;
      const int64_t iq = i0w + n;  // this lane's query
      const bf16x8 bq0 = as_bf8(qh0), bq1 = as_bf8(qh1);

      // ---- logits: window band (keys i0w-16+kappa, kappa < 32) and table entries
      f4 S0 = {0, 0, 0, 0}, S1 = {0, 0, 0, 0};
      {
        const int sa = slot_of(i0w - 16 + n), sb = slot_of(i0w + n);
        S0 = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sa, g))), bq0, S0);
        S0 = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sa, 4 + g))), bq1, S0);
        S1 = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sb, g))), bq0, S1);
        S1 = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sb, 4 + g))), bq1, S1);
      }
      float s_ent[kMaxEnt];
      // covered entries: slabs from the ring
      for (int e = 0; e < a.n_cov; ++e) {
        const int d = a.dist[e];
        const int sl = slot_of(i0w - d + n);
        f4 S = {0, 0, 0, 0};
        S = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sl, g))), bq0, S);
        S = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sl, 4 + g))), bq1, S);
        float s = sel4(S, l);
        if (MODE == 1) {
          const int sh = slot_of(i0w - d + 1 + n);
          f4 H = {0, 0, 0, 0};
          H = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sh, g))), bq0, H);
          H = mfma32(as_bf8(lds_read16(sm.ringK, chunk_off(sh, 4 + g))), bq1, H);
          s = fmaf(a.w[e], sel4(H, l) - s, s);
        }
        s_ent[e] = (diag_lane && (int64_t)d <= iq) ? s * sl2 : -INFINITY;
      }
      // far entries: raw K rows from global memory, relatively rotated queries
      for (int e = a.n_cov; e < a.n_ent; ++e) {
        const int d = a.dist[e];
        const int u = MODE == 1 ? 2 * (e - a.n_cov) : e - a.n_cov;
        float s;
        {
          int64_t r = i0w - d + n;
          r = r < 0 ? 0 : r;
          const bf16_t* kp = Kh + r * kD;
          const uint4 k0 = *reinterpret_cast<const uint4*>(kp + 8 * g);
          const uint4 k1 = *reinterpret_cast<const uint4*>(kp + kHalf + 8 * g);
          uint4 r0, r1;
          rotate_pack(qraw0, qraw1, &sm.unc_cs[u][8 * g], &r0, &r1);
          f4 S = {0, 0, 0, 0};
          S = mfma32(as_bf8(k0), as_bf8(r0), S);
          S = mfma32(as_bf8(k1), as_bf8(r1), S);
          s = sel4(S, l);
        }
        if (MODE == 1) {
          int64_t r = i0w - d + 1 + n;
          r = r < 0 ? 0 : r;
          const bf16_t* kp = Kh + r * kD;
          const uint4 k0 = *reinterpret_cast<const uint4*>(kp + 8 * g);
          const uint4 k1 = *reinterpret_cast<const uint4*>(kp + kHalf + 8 * g);
          uint4 r0, r1;
          rotate_pack(qraw0, qraw1, &sm.unc_cs[u + 1][8 * g], &r0, &r1);
          f4 H = {0, 0, 0, 0};
          H = mfma32(as_bf8(k0), as_bf8(r0), H);
          H = mfma32(as_bf8(k1), as_bf8(r1), H);
          s = fmaf(a.w[e], sel4(H, l) - s, s);
        }
        s_ent[e] = (diag_lane && (int64_t)d <= iq) ? s * sl2 : -INFINITY;
      }

      // ---- softmax over the window band and the entries
      float sw0[4], sw1[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int d0 = n + 16 - 4 * g - v;  // >= 1
        const int d1 = n - 4 * g - v;
        sw0[v] = (d0 < a.W && (int64_t)d0 <= iq) ? S0[v] * sl2 : -INFINITY;
        sw1[v] = (d1 >= 0 && d1 < a.W) ? S1[v] * sl2 : -INFINITY;
      }
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) m = fmaxf(m, fmaxf(sw0[v], sw1[v]));
      for (int e = 0; e < a.n_ent; ++e) m = fmaxf(m, s_ent[e]);
      m = wave_xor_max(m);  // every query has its own key (distance 0), so m is finite
      // lsum (fp32 weights) gives LSE; lnorm sums the bf16 weights the P V products use, so
      // that O is normalised by exactly the weights applied (rows of P sum to 1)
      float lsum = 0.f, lnorm = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sw0[v] = exp2f(sw0[v] - m);
        sw1[v] = exp2f(sw1[v] - m);
        lsum += sw0[v] + sw1[v];
        lnorm += round_bf(sw0[v]) + round_bf(sw1[v]);
      }
      for (int e = 0; e < a.n_ent; ++e) {
        s_ent[e] = exp2f(s_ent[e] - m);
        lsum += s_ent[e];
        if (MODE == 0)
          lnorm += round_bf(s_ent[e]);
        else
          lnorm += round_bf(s_ent[e] * (1.f - a.w[e])) + round_bf(s_ent[e] * a.w[e]);
      }
      lsum = wave_xor_sum(lsum);
      lnorm = wave_xor_sum(lnorm);

      // ---- P V: O^T[dim 16 mb + 4 g + v][query n]
      f4 acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = f4{0, 0, 0, 0};
      const int jr = n >> 2;              // transpose-read row within a 4-row group
      const int jc = n & 3;               // transpose-read 4-column group
      auto tr_off = [&](int64_t row, int mb) {
        const int sl = slot_of(row);
        const int chunk = 2 * mb + (jc >> 1);
        return sl * 128 + ((chunk ^ (sl & 7)) << 4) + ((jc & 1) << 3);
      };
      {
        uint32_t pw[4];
        pw[0] = pack_bf2(sw0[0], sw0[1]);
        pw[1] = pack_bf2(sw0[2], sw0[3]);
        pw[2] = pack_bf2(sw1[0], sw1[1]);
        pw[3] = pack_bf2(sw1[2], sw1[3]);
        const bf16x8 bp = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        const int64_t r0 = i0w - 16 + 4 * g + jr, r1 = i0w + 4 * g + jr;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[mb] = mfma32(cat_bf8(tr16(sm.ringV, tr_off(r0, mb)), tr16(sm.ringV, tr_off(r1, mb))), bp, acc[mb]);
      }
      // stage far V rows (this wave's region), rows i0w - d + r for r < 16 (+1 upper row)
      auto stage_rows = [&](int d) {
        uint8_t* st = sm.stage[wave];
        for (int r = n; r < kStageRows; r += 16) {
          int64_t row = i0w - d + r;
          row = row < 0 ? 0 : (row >= N ? N - 1 : row);
          const bf16_t* vp = Vh + row * kD;
          lds_write16(st, r * 128 + ((g ^ (r & 7)) << 4), *reinterpret_cast<const uint4*>(vp + 8 * g));
          lds_write16(st, r * 128 + (((4 + g) ^ (r & 7)) << 4), *reinterpret_cast<const uint4*>(vp + kHalf + 8 * g));
        }
      };
      auto st_off = [&](int r, int mb) {
        const int chunk = 2 * mb + (jc >> 1);
        return r * 128 + ((chunk ^ (r & 7)) << 4) + ((jc & 1) << 3);
      };
      if (MODE == 0) {
        int e = 0;
        for (; e + 1 < a.n_ent; e += 2) {
          uint32_t d0, d1, d2, d3;
          diag_slots(s_ent[e], l, diag_lane, &d0, &d1);
          diag_slots(s_ent[e + 1], l, diag_lane, &d2, &d3);
          const bf16x8 bp = __builtin_bit_cast(bf16x8, make_uint4(d0, d1, d2, d3));
          const bool far0 = e >= a.n_cov, far1 = e + 1 >= a.n_cov;
          s4 lo[4], hi[4];
          if (far0) {
            stage_rows(a.dist[e]);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) lo[mb] = tr16(sm.stage[wave], st_off(4 * g + jr, mb));
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) lo[mb] = tr16(sm.ringV, tr_off(i0w - a.dist[e] + 4 * g + jr, mb));
          }
          if (far1) {
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
            stage_rows(a.dist[e + 1]);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) hi[mb] = tr16(sm.stage[wave], st_off(4 * g + jr, mb));
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) hi[mb] = tr16(sm.ringV, tr_off(i0w - a.dist[e + 1] + 4 * g + jr, mb));
          }
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma32(cat_bf8(lo[mb], hi[mb]), bp, acc[mb]);
          __builtin_amdgcn_s_waitcnt(0);
          __builtin_amdgcn_wave_barrier();
        }
        if (e < a.n_ent) {
          uint32_t d0, d1;
          diag_slots(s_ent[e], l, diag_lane, &d0, &d1);
          const bf16x4 bp = __builtin_bit_cast(bf16x4, make_uint2(d0, d1));
          if (e >= a.n_cov) {
            stage_rows(a.dist[e]);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[mb] = mfma16(as_bf4(tr16(sm.stage[wave], st_off(4 * g + jr, mb))), bp, acc[mb]);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[mb] = mfma16(as_bf4(tr16(sm.ringV, tr_off(i0w - a.dist[e] + 4 * g + jr, mb))), bp, acc[mb]);
          }
        }
      } else {
        for (int e = 0; e < a.n_ent; ++e) {
          const float w = a.w[e];
          uint32_t d0, d1, d2, d3;
          diag_slots(s_ent[e] * (1.f - w), l, diag_lane, &d0, &d1);
          diag_slots(s_ent[e] * w, l, diag_lane, &d2, &d3);
          const bf16x8 bp = __builtin_bit_cast(bf16x8, make_uint4(d0, d1, d2, d3));
          const int d = a.dist[e];
          if (e >= a.n_cov) {
            stage_rows(d);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[mb] = mfma32(cat_bf8(tr16(sm.stage[wave], st_off(4 * g + jr, mb)),
                                       tr16(sm.stage[wave], st_off(4 * g + jr + 1, mb))), bp, acc[mb]);
            __builtin_amdgcn_s_waitcnt(0);
            __builtin_amdgcn_wave_barrier();
          } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[mb] = mfma32(cat_bf8(tr16(sm.ringV, tr_off(i0w - d + 4 * g + jr, mb)),
                                       tr16(sm.ringV, tr_off(i0w - d + 1 + 4 * g + jr, mb))), bp, acc[mb]);
          }
        }
      }

      // ---- epilogue
      if (iq < s1) {
        const float inv = 1.f / lnorm;
        bf16_t* op = a.o + hoff + iq * kD + 4 * g;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          uint2 x;
          x.x = pack_bf2(acc[mb][0] * inv, acc[mb][1] * inv);
          x.y = pack_bf2(acc[mb][2] * inv, acc[mb][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * mb) = x;
        }
        if (g == 0 && a.lse != nullptr) a.lse[(size_t)head * N + iq] = (m + log2f(lsum)) * 0.69314718055994530942f;
      }
    }
    __syncthreads();
  }
}

// far distances of a table: integer d, or c and c - 1 per interpolated entry
int count_far(const FwdArgs& f, int* n_cov) {
  int cov = 0;
  while (cov < f.tab.n && f.tab.dist[cov] <= kMaxCov) ++cov;
  *n_cov = cov;
  const int far = f.tab.n - cov;
  return f.mode == 1 ? 2 * far : far;
}

}  // namespace

bool fwd_ring_supported(const FwdArgs& f) {
  if (f.dtype != 1 || f.W > kMaxBand) return false;
  int cov;
  return count_far(f, &cov) <= kMaxUnc;
}

hipError_t launch_fwd_ring(const FwdArgs& f) {
  RingArgs a;
  a.q = (const bf16_t*)f.q;
  a.k = (const bf16_t*)f.k;
  a.v = (const bf16_t*)f.v;
  a.o = (bf16_t*)f.o;
  a.lse = f.lse;
  a.N = f.N;
  a.W = f.W;
  a.n_ent = f.tab.n;
  a.n_unc = count_far(f, &a.n_cov);
  for (int e = 0; e < kMaxEnt; ++e) {
    a.dist[e] = f.tab.dist[e];
    a.w[e] = f.tab.w[e];
  }
  int u = 0;
  for (int e = a.n_cov; e < f.tab.n; ++e) {
    a.unc_dist[u++] = f.tab.dist[e];
    if (f.mode == 1) a.unc_dist[u++] = f.tab.dist[e] - 1;
  }
  for (; u < kMaxUnc; ++u) a.unc_dist[u] = 0;
  // rows before a segment start that the ring must hold: the band and the covered distances
  int need = kMaxBand;
  for (int e = 0; e < a.n_cov; ++e) need = f.tab.dist[e] > need ? f.tab.dist[e] : need;
  a.warm = ((need + kT - 1) / kT) * kT;
  // segments: about one workgroup per CU in total
  const int64_t tiles = (f.N + kT - 1) / kT;
  int64_t segs = (256 + f.BH - 1) / f.BH;
  if (segs > tiles) segs = tiles;
  if (segs < 1) segs = 1;
  const int64_t per = (tiles + segs - 1) / segs;
  segs = (tiles + per - 1) / per;
  a.seg_len = (int)(per * kT);
  a.segs = (int)segs;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kD));
  a.rope = f.rope;
  const size_t smem = sizeof(Smem);
  const void* fn = f.mode == 0 ? (const void*)fwd_ring_kernel<0> : (const void*)fwd_ring_kernel<1>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(segs * f.BH)), block(kThreads);
  if (f.mode == 0)
    fwd_ring_kernel<0><<<grid, block, smem, f.stream>>>(a);
  else
    fwd_ring_kernel<1><<<grid, block, smem, f.stream>>>(a);
  return hipGetLastError();
}

}  // namespace fib
