// Query side of the backward pass on the LDS ring (bf16, D = 64, W <= 16, integer and
// interpolated offsets): dQ, Delta and the per-workgroup partials of d(alpha).
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science summaries
// of arXiv 2606.28560, Method > Architecture and attention mechanism; the interpolated rows
// exist so that the Learned schedule of Method > Experimental variables can train alpha):
// with s = <R_i q_i, key>/sqrt(D), P = exp(s - LSE_i), Delta_i = <dO_i, O_i>,
// dP = <dO_i, value>, dS = P (dP - Delta_i),
//   dQ_i = R_i^T sum dS key^ / sqrt(D)           (key^ the rotated key; R_i^T undoes RoPE)
//   dalpha += -f [dS (s_hi - s_lo) + P <dO_i, v_hi - v_lo>]   (interpolated entries)
//
// Design: the forward's ring (fwd_ring.hip) with a second operand set. Per step each wave
// takes 16 queries; the ring holds K^ and V (both in natural dim order). Logits S^T = K^ Q^T
// and dP^T = V dO^T on MFMA (window band: 32 keys x 16 queries; a table entry: a 16-row slab
// whose diagonal is used), P from the stored LSE (no max), dS on VALU, then
// dQ^T = K^T dS^T on MFMA, K^T read from the ring through the transpose read with addresses
// chosen so that lane (n, g) accumulates dims 8g..8g+7 and 32+8g..32+8g+7 of query n: the
// same dims whose RoPE angles it computed for the insert, so it undoes R_i in registers. Far
// entries (beyond the ring) read K and V rows from global memory, their dP a VALU dot. In
// interpolated mode the kernel writes every rotated row R_i q_i and R_j k_j of its segment to
// the workspace (the key side, bound there by its VALU work, reads them instead of rotating
// its own; the integer mode, bound by its memory traffic, does without the writes). Far K
// rows: either those rotated rows (ROT instances, interpolated mode; the workgroup first
// writes the rotated rows before its segment that its far entries read), whose logits are
// then an MFMA with the rotated queries and whose dQ contribution dS k^ joins the rotated
// frame before R_i is undone; or raw K rows, with the relative rotation <R_d q, k> for the
// logits and dS R_(-d) k added in the un-rotated frame.
#include "ring_common.h"

#include <algorithm>

namespace fib {
namespace {

using namespace ring;

struct BqArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* o;
  const bf16_t* dout;
  const float* lse;
  bf16_t* dq;
  float* delta;
  float* dalpha_part;  // one per workgroup (interpolated mode)
  uint32_t* ps;        // interpolated mode: (P, dS) (ps_pack) per [head][entry][query], or null
  int ps_slots;        // entries per head in ps
  bf16_t* qr;          // interpolated: rotated rows R_i q_i, [head][N][D] (written)
  bf16_t* kr;          // interpolated: rotated rows R_j k_j, [head][N][D] (written; ROT instances also read them)
  int far_reach;       // the largest far distance in use (ROT instances; DEV: from the plan)
  int N;
  int W;
  int n_cov;
  int early_rows;
  int seg_len;
  int segs;
  int warm;
  float scale;       // 1 / sqrt(D)
  float scale_log2;  // scale * log2(e)
  int dist[kMaxCov];
  float w[kMaxCov];
  float f[kMaxCov];
  int far_dist[kMaxFar];
  float far_w[kMaxFar];
  float far_f[kMaxFar];
  int unc_dist[kMaxUnc];
  Rope rope;
  const DevPlan* plan;  // alpha in device memory: the split above comes from here (DEV instances)
  int n_far;            // far entries in use (DEV instances: NF is an upper bound)
  int heads_per_plan;   // DEV instances: head h reads plan[h / heads_per_plan]
};

struct __align__(16) BqSmem {
  uint8_t ringK[(kP + kMirror) * kRow];
  uint8_t ringV[(kP + kMirror) * kRow];
  float2 unc_cs[kMaxUnc][kHalf];
  float2 base_cs[2][kHalf];
  float2 warm_cs[8][kHalf];
  float red[16];
};

// Rows of the far entries for the wave's queries i0w + n, of K or V: lane (n, g) holds row
// i0w - d + n (the lower row in interpolated mode), dims 8g..8g+7 and 32+8g..32+8g+7. In
// interpolated mode the upper row of query n is the lower row of query n + 1 (upper_rows);
// the one that no lane holds, row i0w - d + 16, is kept spread over the wave, lane l holding
// its dword l % 32.
template <int MODE, int NF>
struct FarK {
  uint4 k[NF > 0 ? NF : 1][2];
  uint32_t ex[MODE == 1 && NF > 0 ? NF : 1];
};

// n_use: far slots to load (the rest are zero-filled). The kernel passes NF: in DEV
// instances the unused slots load in-bounds rows and are masked, since skipping their loads
// by a branch costs this kernel its register fit.
template <int MODE, int NF>
__device__ __forceinline__ void load_far(const int* fdist, int n_use, FarK<MODE, NF>& fr, const BqArgs& a,
                                         const bf16_t* X, int i0w, int l, int n, int g, int lane_off) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f >= n_use) {
      fr.k[f][0] = fr.k[f][1] = make_uint4(0, 0, 0, 0);
      if constexpr (MODE == 1) fr.ex[f] = 0u;
      continue;
    }
    const bf16_t* p = X + far_off(fdist[f], i0w, n, g, lane_off);
    fr.k[f][0] = *reinterpret_cast<const uint4*>(p);
    fr.k[f][1] = *reinterpret_cast<const uint4*>(p + kHalf);
    if constexpr (MODE == 1) {
      // row i0w - d + 16 (< N: far distances exceed 16); rows before 0 only meet masked queries
      const int r = i0w - fdist[f] + 16;
      fr.ex[f] = reinterpret_cast<const uint32_t*>(X + (int64_t)(r > 0 ? r : 0) * kD)[l & 31];
    }
  }
}

// <x, y> over the lane's 16 dims of two packed bf16 rows (fp32 accumulation)
__device__ __forceinline__ float dot16_bf(uint4 x0, uint4 x1, uint4 y0, uint4 y1) {
  float s = dot2(x0.x, y0.x, 0.f);
  s = dot2(x0.y, y0.y, s);
  s = dot2(x0.z, y0.z, s);
  s = dot2(x0.w, y0.w, s);
  s = dot2(x1.x, y1.x, s);
  s = dot2(x1.y, y1.y, s);
  s = dot2(x1.z, y1.z, s);
  return dot2(x1.w, y1.w, s);
}

// acc (dims 8g+t in lo[t], 32+8g+t in hi[t]) += c * R_(-d) x for a raw packed row x, with
// cs[t] = (cos, sin) of d * omega_(8g+t)
__device__ __forceinline__ void add_unrot(float* lo, float* hi, float c, uint4 x0, uint4 x1, const float2* cs) {
  float xf[16];
  unpack8(x0, xf);
  unpack8(x1, xf + 8);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    lo[t] = fmaf(c, xf[t] * cs[t].x + xf[8 + t] * cs[t].y, lo[t]);
    hi[t] = fmaf(c, xf[8 + t] * cs[t].x - xf[t] * cs[t].y, hi[t]);
  }
}

// acc (the rotated frame: dims 8g+t in acc[t / 4][t % 4], 32+8g+t in acc[2 + t / 4][t % 4])
// += c * x for a packed rotated row x
__device__ __forceinline__ void add_rot(f4* acc, float c, uint4 x0, uint4 x1) {
  float xf[16];
  unpack8(x0, xf);
  unpack8(x1, xf + 8);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    acc[t >> 2][t & 3] = fmaf(c, xf[t], acc[t >> 2][t & 3]);
    acc[2 + (t >> 2)][t & 3] = fmaf(c, xf[8 + t], acc[2 + (t >> 2)][t & 3]);
  }
}

// (cos, sin) of the angle sum of two (cos, sin) pairs, with the operations spelled out: the
// warm-up and the step loop rotate the same rows and must round them identically
__device__ __forceinline__ float2 compose_cs(float2 b, float2 t) {
  return make_float2(fmaf(b.x, t.x, -(b.y * t.y)), fmaf(b.y, t.x, b.x * t.y));
}
// R x of 16 unpacked values (pairs (x[t], x[8 + t])), packed bf16 halves; spelled out as
// compose_cs
__device__ __forceinline__ void rotate_pack_x(const float* x, const float2* cs, uint4* out_lo, uint4* out_hi) {
  float ra[8], rb[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    ra[t] = fmaf(x[t], cs[t].x, -(x[8 + t] * cs[t].y));
    rb[t] = fmaf(x[8 + t], cs[t].x, x[t] * cs[t].y);
  }
  *out_lo = pack8(ra);
  *out_hi = pack8(rb);
}

template <int MODE, int NC, int NF, int WAVES, bool DEV, bool ROT>
__global__ __launch_bounds__(64 * WAVES, 1) void bwdq_ring_kernel(BqArgs a) {
  constexpr int kThreads = 64 * WAVES;
  constexpr int kT = step_rows(WAVES);
  extern __shared__ __align__(16) uint8_t smem_raw[];
  BqSmem& sm = *reinterpret_cast<BqSmem*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int n = l & 15;
  const int g = l >> 4;
  const bool diag_lane = g == (n >> 2);
  const int jr = n >> 2;
  const int jc = n & 3;
  const int N = a.N;
  const float log2e = 1.4426950408889634f;
  // alpha-dependent launch data: the kernel arguments, or (DEV instances, alpha in device
  // memory) the split built on the device, read once into registers (the arguments struct
  // itself is never written, so it stays in the kernel-argument segment)
  RingSplit lcl;
  const DevPlan* pl = a.plan;
  if constexpr (DEV) {
    pl += (int)(blockIdx.x / a.segs) / a.heads_per_plan;
    lcl = (WAVES == 8 ? pl->s8 : pl->s4);
  }
  const int S_n_cov = DEV ? lcl.n_cov : a.n_cov;
  const int S_n_far = DEV ? lcl.n_far : a.n_far;
  const int S_early_rows = DEV ? lcl.early_rows : a.early_rows;
  const int S_warm = DEV ? ((lcl.need + kT - 1) / kT) * kT : a.warm;
  auto S_dist = [&](int x) -> int { if constexpr (DEV) return lcl.dist[x]; else return a.dist[x]; };
  auto S_w = [&](int x) -> float { if constexpr (DEV) return lcl.w[x]; else return a.w[x]; };
  auto S_f = [&](int x) -> float { if constexpr (DEV) return lcl.f[x]; else return a.f[x]; };
  auto S_far_dist = [&](int x) -> int { if constexpr (DEV) return lcl.far_dist[x]; else return a.far_dist[x]; };
  auto S_far_w = [&](int x) -> float { if constexpr (DEV) return lcl.far_w[x]; else return a.far_w[x]; };
  auto S_far_f = [&](int x) -> float { if constexpr (DEV) return lcl.far_f[x]; else return a.far_f[x]; };
  // (DEV: over every far slot the kernel loads, the unused ones included)
  int S_far_reach = a.far_reach;
  if constexpr (DEV) {
    S_far_reach = 0;
#pragma unroll
    for (int f = 0; f < NF; ++f) S_far_reach = lcl.far_dist[f] > S_far_reach ? lcl.far_dist[f] : S_far_reach;
  }


  {
    constexpr int n_unc = MODE == 1 ? 2 * NF : NF;
    for (int x = tid; x < n_unc * kHalf; x += kThreads) {
      const int u = x / kHalf, j = x % kHalf;
      int d;
      if constexpr (DEV) d = (WAVES == 8 ? pl->s8 : pl->s4).unc_dist[u];
      else d = a.unc_dist[u];  // (a's arrays are indexed by constants only in DEV instances)
      sm.unc_cs[u][j] = rope_cs(d, a.rope.rev[j]);
    }
  }
  float2 cs_t[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) cs_t[t] = rope_cs(16 * wave + n, a.rope.rev[8 * g + t]);
  // the lane's inverse frequency for the per-step base rotation (wave 0, lanes < 32), read once:
  // indexed per lane, it is a memory load, and inside the step loop its wait would also wait
  // for the next step's rows requested just before it
  const double rev_l = a.rope.rev[l & (kHalf - 1)];
  const float sl2 = a.scale_log2;
  // Lane constants formed anew in every step (a few VALU operations) rather than held in
  // registers through the loop: the window masks (band key kappa of the lane at distance
  // n + 16 - 4g - v in block 0 and n - 4g - v in block 1) and the selectors of diag_block.
  // (The empty asm makes W and the lane opaque, so the compiler does not hoist them.) Masks
  // select -inf instead of adding it, so a NaN logit of an unattended key stays masked.
  auto window_in = [&](bool* in0, bool* in1) {
    int Wp = a.W;
    asm volatile("" : "+s"(Wp));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int d0 = n + 16 - 4 * g - v, d1 = n - 4 * g - v;
      in0[v] = d0 < Wp;
      in1[v] = d1 >= 0 && d1 < Wp;
    }
  };
  auto diag_sel = [&](uint32_t* sel) {
    int lp = l;
    asm volatile("" : "+v"(lp));
    const uint32_t zero = 0x0c0c0c0cu;
    const uint32_t a_half = (lp & 1) ? 0x01000c0cu : 0x0c0c0100u;
    const uint32_t b_half = (lp & 1) ? 0x03020c0cu : 0x0c0c0302u;
    const bool low = (lp & 2) == 0;
    sel[0] = low ? a_half : zero;
    sel[1] = low ? zero : a_half;
    sel[2] = low ? b_half : zero;
    sel[3] = low ? zero : b_half;
  };
  const int diag_addr = 4 * (16 * (n >> 2) + n);
  const int lane_k = n * kRow + 16 * g;
  // transpose reads of K^: lane (jr, jc) of group g reads row 4g + jr at dims 8 jc + 4 h +
  // 32 h2 (output block mb = 2 h2 + h), so output row 4g' + v of block mb is dim
  // 8g' + 4h + 32h2 + v
  const int lane_t = (4 * g + jr) * kRow + 16 * jc;
  const int lane_off = n * kD + 8 * g;

  const int64_t head = blockIdx.x / a.segs;
  const int seg = blockIdx.x % a.segs;
  const int s0 = seg * a.seg_len;
  const int s1 = s0 + a.seg_len < N ? s0 + a.seg_len : N;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const bf16_t* Qh = a.q + hoff;
  const bf16_t* Kh = a.k + hoff;
  const bf16_t* Vh = a.v + hoff;
  const bf16_t* Oh = a.o + hoff;
  const bf16_t* Dh = a.dout + hoff;
  const float* Lh = a.lse + (size_t)head * N;
  bf16_t* QRh = MODE == 1 ? a.qr + hoff : nullptr;
  bf16_t* KRh = MODE == 1 ? a.kr + hoff : nullptr;
  // the far entries' K rows: rotated (ROT) or raw
  const bf16_t* Fh = ROT ? KRh : Kh;

  // stores row rb + n of the lane: K^ and V, both in natural dim order
  auto put_row = [&](int rb, uint4 k0, uint4 k1, uint4 v0, uint4 v1) {
    const int slot = rb & (kP - 1);
    auto put = [&](int ro) {
      lds_write16(sm.ringK + ro + 16 * g, 0, k0);
      lds_write16(sm.ringK + ro + 16 * g, 64, k1);
      lds_write16(sm.ringV + ro + 16 * g, 0, v0);
      lds_write16(sm.ringV + ro + 16 * g, 64, v1);
    };
    put((slot + n) * kRow);
    if (slot < kMirror) put((slot + kP + n) * kRow);
  };
  // element offset of the lane's part of row rb + n (rows past the end repeat row N - 1)
  auto row_elems = [&](int rb) -> int64_t {
    if (rb + 15 < N) return (int64_t)rb * kD + lane_off;
    const int r = rb + n < N ? rb + n : N - 1;
    return (int64_t)r * kD + 8 * g;
  };
  auto load2 = [&](const bf16_t* base, int64_t off, uint4* x) {
    x[0] = *reinterpret_cast<const uint4*>(base + off);
    x[1] = *reinterpret_cast<const uint4*>(base + off + kHalf);
  };
  // the lane's part of row rb + n of a rotated-row buffer (a wave-uniform row base plus the
  // lane's 32-bit byte offset, made opaque so that no per-lane 64-bit address is held)
  auto put_rot = [&](bf16_t* base, int rb, uint4 x0, uint4 x1) {
    char* b = reinterpret_cast<char*>(base + (int64_t)rb * kD);
    uint32_t lb = 2u * (uint32_t)lane_off;
    asm volatile("" : "+v"(lb));
    *reinterpret_cast<uint4*>(b + lb) = x0;
    *reinterpret_cast<uint4*>(b + lb + 2 * kHalf) = x1;
  };

  // ---- warm-up (as in the forward): ring rows [ws, s0)
  const int ws = s0 - S_warm > 0 ? s0 - S_warm : 0;
  const int n_warm = (s0 - ws) / kT;
  if (s0 < S_warm) {
    uint4* z = reinterpret_cast<uint4*>(sm.ringK);
    const int n16 = (2 * (kP + kMirror) * kRow) / 16;
    for (int x = tid; x < n16; x += kThreads) z[x] = make_uint4(0, 0, 0, 0);
  }
  if (tid < kHalf * (n_warm + 1)) {
    const int j = tid / kHalf, t = tid % kHalf;
    if (j < n_warm) sm.warm_cs[j][t] = rope_cs(ws + j * kT, a.rope.rev[t]);
    else sm.base_cs[0][t] = rope_cs(s0, a.rope.rev[t]);
  }
  uint4 pq[2], pk[2], pv[2], pd[2];
  float plse;
  {
    const int64_t off = row_elems(s0 + 16 * wave);
    load2(Qh, off, pq);
    load2(Kh, off, pk);
    load2(Vh, off, pv);
    load2(Dh, off, pd);
    const int r = s0 + 16 * wave + n;
    plse = Lh[r < N ? r : N - 1];
  }
  __syncthreads();
  {
    constexpr int kWB = WAVES == 8 ? 3 : 4;
    for (int j0 = 0; j0 < n_warm; j0 += kWB) {
      uint4 wk[kWB][2], wv[kWB][2];
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          const int64_t off = (int64_t)(ws + (j0 + jj) * kT + 16 * wave) * kD + lane_off;
          load2(Kh, off, wk[jj]);
          load2(Vh, off, wv[jj]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          float2 cs[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) cs[t] = compose_cs(sm.warm_cs[j0 + jj][8 * g + t], cs_t[t]);
          float kf[16];
          unpack8(wk[jj][0], kf);
          unpack8(wk[jj][1], kf + 8);
          uint4 kr0, kr1;
          rotate_pack_x(kf, cs, &kr0, &kr1);
          put_row(ws + (j0 + jj) * kT + 16 * wave, kr0, kr1, wv[jj][0], wv[jj][1]);
          // (the far entries of the first steps read these rows, which precede the segment)
          if constexpr (ROT) put_rot(KRh, ws + (j0 + jj) * kT + 16 * wave, kr0, kr1);
        }
      }
    }
  }
  if constexpr (ROT) {
    // the rotated rows [s0 - far_reach, ws) that the far entries read before the step loop
    // has written them (rows of the previous segment; its workgroup writes the same values)
    const int xs = s0 - S_far_reach > 0 ? s0 - S_far_reach : 0;
    const int n_ext = ws > xs ? (ws - xs + kT - 1) / kT : 0;  // 128-row blocks below ws
    for (int j0 = 0; j0 < n_ext; j0 += 8) {
      __syncthreads();  // (warm_cs is reused)
      if (tid < kHalf * 8) {
        const int j = tid / kHalf, t = tid % kHalf;
        if (j0 + j < n_ext) sm.warm_cs[j][t] = rope_cs(ws - (j0 + j + 1) * kT, a.rope.rev[t]);
      }
      __syncthreads();
      for (int jj = 0; jj < 8 && j0 + jj < n_ext; ++jj) {
        const int rb = ws - (j0 + jj + 1) * kT + 16 * wave;
        if (rb + 15 >= xs) {
          const int r = rb + n >= 0 ? rb + n : 0;
          uint4 xk[2];
          load2(Kh, (int64_t)r * kD + 8 * g, xk);
          float2 cs[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) cs[t] = compose_cs(sm.warm_cs[jj][8 * g + t], cs_t[t]);
          float kf[16];
          unpack8(xk[0], kf);
          unpack8(xk[1], kf + 8);
          uint4 kr0, kr1;
          rotate_pack_x(kf, cs, &kr0, &kr1);
          if (rb + n >= 0) put_rot(KRh, rb, kr0, kr1);
        }
      }
    }
    // the first segment's far rows before the step loop are all row 0 (clamped): its rotation,
    // as the first step's insert forms it
    if (s0 == 0 && wave == 0) {
      uint4 xk[2];
      load2(Kh, (int64_t)(n < N ? n : N - 1) * kD + 8 * g, xk);
      float2 cs[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) cs[t] = compose_cs(sm.base_cs[0][8 * g + t], cs_t[t]);
      float kf[16];
      unpack8(xk[0], kf);
      unpack8(xk[1], kf + 8);
      uint4 kr0, kr1;
      rotate_pack_x(kf, cs, &kr0, &kr1);
      if (n < N) put_rot(KRh, 0, kr0, kr1);
    }
    // the rows written above and in the warm-up are read by other waves after this
    __syncthreads();
  }
  FarK<MODE, NF> fk;
  load_far<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, NF, fk, a, Fh, s0 + 16 * wave, l, n, g, lane_off);
  float dal = 0.f;  // d(alpha) contributions of this lane's queries

  int buf = 0;
  for (int p0 = s0; p0 < s1; p0 += kT, buf ^= 1) {
    // ---- insert: K^ and V of rows p0 + 16w + n; rotated Q of the step's queries
    float2 cs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) cs[t] = compose_cs(sm.base_cs[buf][8 * g + t], cs_t[t]);
    float qf[16];
    uint4 qh0, qh1;
    {
      float kf[16];
      unpack8(pq[0], qf);
      unpack8(pq[1], qf + 8);
      unpack8(pk[0], kf);
      unpack8(pk[1], kf + 8);
      uint4 kr0, kr1;
      rotate_pack_x(kf, cs, &kr0, &kr1);
      rotate_pack_x(qf, cs, &qh0, &qh1);
      put_row(p0 + 16 * wave, kr0, kr1, pv[0], pv[1]);
      // the segment's rotated rows, for the key side (and the far entries of later steps)
      if (MODE == 1 && p0 + 16 * wave + n < s1) {
        put_rot(KRh, p0 + 16 * wave, kr0, kr1);
        put_rot(QRh, p0 + 16 * wave, qh0, qh1);
      }
    }
    const uint4 do0 = pd[0], do1 = pd[1];
    const float lse2 = plse * log2e;
    __syncthreads();
    const int pn = p0 + kT;
    // the next step's rows (this step's were consumed by the insert above). Integer mode
    // requests them here, a whole step ahead; interpolated mode, whose steps are twice as
    // long, after the covered entries, so that their 33 registers are not held through the
    // step's register peak (held, they cost spills whose reloads wait for every load in
    // flight)
    auto prefetch = [&]() {
      const int pr = pn < s1 ? pn : p0;
      const int64_t off = row_elems(pr + 16 * wave);
      load2(Qh, off, pq);
      load2(Kh, off, pk);
      load2(Vh, off, pv);
      load2(Dh, off, pd);
      const int r = pr + 16 * wave + n;
      plse = Lh[r < N ? r : N - 1];
    };
    if constexpr (MODE == 0) prefetch();
    if (wave == 0 && l < kHalf) sm.base_cs[buf ^ 1][l] = rope_cs(pn, rev_l);

    const int bw = p0 + 16 * wave;
    const int i0w = bw;
    const int iq = i0w + n;
    const bool early = i0w < S_early_rows;
    // O rows of the step's queries, for Delta (used after the logits)
    uint4 oo[2];
    load2(Oh, row_elems(i0w), oo);
    const bf16x8 bq0 = as_bf8(qh0), bq1 = as_bf8(qh1);
    const bf16x8 bd0 = as_bf8(do0), bd1 = as_bf8(do1);

    // ---- window band: logits and dP for keys i0w - 16 + kappa
    const int band = row_off(bw - 16);
    f4 S0 = {0, 0, 0, 0}, S1 = {0, 0, 0, 0}, D0 = {0, 0, 0, 0}, D1 = {0, 0, 0, 0};
    {
      const int sa = band + lane_k;
      S0 = mfma32(as_bf8(lds_read16(sm.ringK, sa)), bq0, S0);
      S0 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 64)), bq1, S0);
      S1 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 16 * kRow)), bq0, S1);
      S1 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 16 * kRow + 64)), bq1, S1);
      D0 = mfma32(as_bf8(lds_read16(sm.ringV, sa)), bd0, D0);
      D0 = mfma32(as_bf8(lds_read16(sm.ringV, sa + 64)), bd1, D0);
      D1 = mfma32(as_bf8(lds_read16(sm.ringV, sa + 16 * kRow)), bd0, D1);
      D1 = mfma32(as_bf8(lds_read16(sm.ringV, sa + 16 * kRow + 64)), bd1, D1);
    }
    // ---- covered entries: logits and dP (interpolated: lower and upper slab)
    float s_e[NC], dp_e[NC], sd_e[MODE == 1 ? NC : 1], dd_e[MODE == 1 ? NC : 1];
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      const int sl = row_off(bw - S_dist(e)) + lane_k;
      f4 S = {0, 0, 0, 0}, P = {0, 0, 0, 0};
      S = mfma32(as_bf8(lds_read16(sm.ringK, sl)), bq0, S);
      S = mfma32(as_bf8(lds_read16(sm.ringK, sl + 64)), bq1, S);
      P = mfma32(as_bf8(lds_read16(sm.ringV, sl)), bd0, P);
      P = mfma32(as_bf8(lds_read16(sm.ringV, sl + 64)), bd1, P);
      s_e[e] = sel4(S, l);
      dp_e[e] = sel4(P, l);
      if (MODE == 1) {
        f4 H = {0, 0, 0, 0}, Q = {0, 0, 0, 0};
        H = mfma32(as_bf8(lds_read16(sm.ringK, sl + kRow)), bq0, H);
        H = mfma32(as_bf8(lds_read16(sm.ringK, sl + kRow + 64)), bq1, H);
        Q = mfma32(as_bf8(lds_read16(sm.ringV, sl + kRow)), bd0, Q);
        Q = mfma32(as_bf8(lds_read16(sm.ringV, sl + kRow + 64)), bd1, Q);
        sd_e[e] = sel4(H, l) - s_e[e];  // s_hi - s_lo
        dd_e[e] = sel4(Q, l) - dp_e[e];  // dp_hi - dp_lo
      }
    }
    // ---- far entries: logits (relative RoPE); their V rows for dP are requested now
    float s_f[NF > 0 ? NF : 1], sd_f[NF > 0 ? NF : 1];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int u = MODE == 1 ? 2 * f : f;
      // the query operand: the rotated query against rotated rows (ROT), else R_d q
      uint4 r0 = qh0, r1 = qh1;
      if constexpr (!ROT) rotate_pack_f(qf, &sm.unc_cs[u][8 * g], &r0, &r1);
      f4 S = {0, 0, 0, 0};
      S = mfma32(as_bf8(fk.k[f][0]), as_bf8(r0), S);
      S = mfma32(as_bf8(fk.k[f][1]), as_bf8(r1), S);
      s_f[f] = sel4(S, l);
      if (MODE == 1) {
        if constexpr (!ROT) rotate_pack_f(qf, &sm.unc_cs[u + 1][8 * g], &r0, &r1);
        uint4 kh[2];
        upper_rows(fk.k[f], fk.ex[f], g, kh);
        f4 H = {0, 0, 0, 0};
        H = mfma32(as_bf8(kh[0]), as_bf8(r0), H);
        H = mfma32(as_bf8(kh[1]), as_bf8(r1), H);
        sd_f[f] = sel4(H, l) - s_f[f];
      }
    }
    FarK<MODE, NF> fv;
    load_far<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, NF, fv, a, Vh, i0w, l, n, g, lane_off);

    // ---- P, Delta, dS
    const float dlt = quad_add(dot16_bf(do0, do1, oo[0], oo[1]));
    float bds[8];  // band dS: sw0 (slab 0) then sw1 (slab 1), per the lane's 4 keys each
    bool in0[4], in1[4];
    window_in(in0, in1);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float x0 = in0[v] ? S0[v] * sl2 : -INFINITY, x1 = in1[v] ? S1[v] * sl2 : -INFINITY;
      if (early && n + 16 - 4 * g - v > iq) x0 = -INFINITY;
      const float p0v = ex2(x0 - lse2), p1v = ex2(x1 - lse2);
      bds[v] = p0v * (D0[v] - dlt);
      bds[4 + v] = p1v * (D1[v] - dlt);
    }
    float dal_step = 0.f;  // this step's d(alpha) terms of the lane's query
    float ds_e[NC];
    uint32_t ps_e[MODE == 1 ? NC : 1];  // interpolated: (P, dS) of each entry, stored at the end
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      float s = s_e[e], dp = dp_e[e];
      if (MODE == 1) {
        s = fmaf(S_w(e), sd_e[e], s);
        dp = fmaf(S_w(e), dd_e[e], dp);
      }
      float x = diag_lane ? s * sl2 : -INFINITY;
      if (e >= S_n_cov || (early && S_dist(e) > iq)) x = -INFINITY;
      const float p = ex2(x - lse2);
      ds_e[e] = p * (dp - dlt);
      if (MODE == 1) {
        dal_step = fmaf(-S_f(e), ds_e[e] * a.scale * sd_e[e] + p * dd_e[e], dal_step);
        ps_e[e] = ps_pack(p, ds_e[e]);
      }
    }

    // ---- dQ^ = K^T dS^T (rotated frame) on MFMA: band, then covered entries
    uint32_t sel[4];
    diag_sel(sel);
    f4 acc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mb] = f4{0, 0, 0, 0};
    {
      const bf16x8 bp = __builtin_bit_cast(
          bf16x8, make_uint4(pack_bf2(bds[0], bds[1]), pack_bf2(bds[2], bds[3]), pack_bf2(bds[4], bds[5]),
                             pack_bf2(bds[6], bds[7])));
      const int r0 = band + lane_t, r1 = r0 + 16 * kRow;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int o = 8 * (mb & 1) + 64 * (mb >> 1);
        acc[mb] = mfma32(cat_bf8(tr16(sm.ringK, r0 + o), tr16(sm.ringK, r1 + o)), bp, acc[mb]);
      }
    }
    if (MODE == 0) {
#pragma unroll
      for (int e = 0; e < NC; e += 2) {
        const bf16x8 bp = diag_block(pack_bf2(ds_e[e], ds_e[e + 1]), sel);
        const int ra = row_off(bw - S_dist(e)) + lane_t, rb = row_off(bw - S_dist(e + 1)) + lane_t;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int o = 8 * (mb & 1) + 64 * (mb >> 1);
          acc[mb] = mfma32(cat_bf8(tr16(sm.ringK, ra + o), tr16(sm.ringK, rb + o)), bp, acc[mb]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        const float ds = ds_e[e];
        const bf16x8 bp = diag_block(pack_bf2(ds * (1.f - S_w(e)), ds * S_w(e)), sel);
        const int ra = row_off(bw - S_dist(e)) + lane_t, rb = ra + kRow;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int o = 8 * (mb & 1) + 64 * (mb >> 1);
          acc[mb] = mfma32(cat_bf8(tr16(sm.ringK, ra + o), tr16(sm.ringK, rb + o)), bp, acc[mb]);
        }
      }
    }
    if constexpr (MODE == 1) prefetch();
    float ql[8], qhv[8];
    // ---- far entries: dP on VALU, P from the diagonal lane, dS; dQ in the rotated frame
    // (ROT: before R_i is undone) or in the un-rotated frame (after)
    uint32_t ps_f[MODE == 1 && NF > 0 ? NF : 1];
    auto far_terms = [&]() {
      if constexpr (MODE == 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int u = MODE == 1 ? 2 * f : f;
        float s = s_f[f];
        if (MODE == 1) s = fmaf(S_far_w(f), sd_f[f], s);
        float x = diag_lane ? s * sl2 : -INFINITY;
        if (early && S_far_dist(f) > iq) x = -INFINITY;
        if (DEV && f >= S_n_far) x = -INFINITY;  // slot beyond the table
        // P of the query, from its diagonal lane to all four
        const float p = __uint_as_float(
            (uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)__float_as_uint(ex2(x - lse2))));
        const float dp_lo = quad_add(dot16_bf(do0, do1, fv.k[f][0], fv.k[f][1]));
        if (MODE == 0) {
          const float ds = p * (dp_lo - dlt);
          if constexpr (ROT) add_rot(acc, ds, fk.k[f][0], fk.k[f][1]);
          else add_unrot(ql, qhv, ds, fk.k[f][0], fk.k[f][1], &sm.unc_cs[u][8 * g]);
        } else {
          uint4 vh[2], kh[2];
          upper_rows(fv.k[f], fv.ex[f], g, vh);
          const float dp_hi = quad_add(dot16_bf(do0, do1, vh[0], vh[1]));
          const float w = S_far_w(f);
          const float ds = p * (fmaf(w, dp_hi - dp_lo, dp_lo) - dlt);
          if constexpr (ROT) add_rot(acc, ds * (1.f - w), fk.k[f][0], fk.k[f][1]);
          else add_unrot(ql, qhv, ds * (1.f - w), fk.k[f][0], fk.k[f][1], &sm.unc_cs[u][8 * g]);
          upper_rows(fk.k[f], fk.ex[f], g, kh);
          if constexpr (ROT) add_rot(acc, ds * w, kh[0], kh[1]);
          else add_unrot(ql, qhv, ds * w, kh[0], kh[1], &sm.unc_cs[u + 1][8 * g]);
          // the diagonal lane holds s_hi - s_lo of its query
          if (diag_lane) dal_step = fmaf(-S_far_f(f), ds * a.scale * sd_f[f] + p * (dp_hi - dp_lo), dal_step);
          ps_f[f] = ps_pack(p, ds);
        }
      }
    };
    if constexpr (ROT) far_terms();
    // undo R_i: dims 8g+t (acc[0], acc[1]) pair with 32+8g+t (acc[2], acc[3])
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float x = acc[t >> 2][t & 3], y = acc[2 + (t >> 2)][t & 3];
      ql[t] = x * cs[t].x + y * cs[t].y;
      qhv[t] = y * cs[t].x - x * cs[t].y;
    }
    if constexpr (!ROT) far_terms();

    // ---- epilogue: dQ = scale * (the lane's 16 dims), Delta
    if constexpr (MODE == 1) {
      // (empty asm: the sums are formed here, not sunk into the conditional stores below)
#pragma unroll
      for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(ql[t]), "+v"(qhv[t]));
    }
    if (iq < s1) {
      // (a wave-uniform row base plus the lane's 32-bit byte offset, made opaque here so that
      // the compiler does not form a per-lane 64-bit address before the loop and hold it)
      char* dp = reinterpret_cast<char*>(a.dq + hoff + (int64_t)i0w * kD);
      uint32_t lb = 2u * (uint32_t)lane_off;
      asm volatile("" : "+v"(lb));
      uint4 x0, x1;
      x0.x = pack_bf2(ql[0] * a.scale, ql[1] * a.scale);
      x0.y = pack_bf2(ql[2] * a.scale, ql[3] * a.scale);
      x0.z = pack_bf2(ql[4] * a.scale, ql[5] * a.scale);
      x0.w = pack_bf2(ql[6] * a.scale, ql[7] * a.scale);
      x1.x = pack_bf2(qhv[0] * a.scale, qhv[1] * a.scale);
      x1.y = pack_bf2(qhv[2] * a.scale, qhv[3] * a.scale);
      x1.z = pack_bf2(qhv[4] * a.scale, qhv[5] * a.scale);
      x1.w = pack_bf2(qhv[6] * a.scale, qhv[7] * a.scale);
      *reinterpret_cast<uint4*>(dp + lb) = x0;
      *reinterpret_cast<uint4*>(dp + lb + 2 * kHalf) = x1;
      if (g == 0) (a.delta + (size_t)head * N + i0w)[n] = dlt;
      dal += dal_step;  // rows past the segment's end belong to another workgroup
      if (MODE == 1 && a.ps != nullptr && diag_lane) {
        // (P, dS) per entry, entry-major: the 16 queries of a wave are 64 contiguous bytes
        uint32_t* pq = a.ps + (size_t)head * a.ps_slots * N + iq;
#pragma unroll
        for (int e = 0; e < NC; ++e)
          if (e < S_n_cov) pq[(size_t)e * N] = ps_e[e];
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (!DEV || f < S_n_far) pq[(size_t)(S_n_cov + f) * N] = ps_f[f];  // (DEV: NF bounds the far count)
      }
    }
    load_far<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, NF, fk, a, Fh, i0w + kT, l, n, g, lane_off);
    __syncthreads();
  }
  if (MODE == 1) {
    // d(alpha) partial of the workgroup: fixed-order sums (wave, then across waves)
    float x = dal;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if (l == 0) sm.red[wave] = x;
    __syncthreads();
    if (tid == 0) {
      float t = 0.f;
      for (int w8 = 0; w8 < WAVES; ++w8) t += sm.red[w8];
      a.dalpha_part[blockIdx.x] = t;
    }
  }
}

// Instances that fit 256 registers per lane, i.e. two waves per SIMD (8 waves); the others
// (16 covered and 4 far entries) run with 4 waves.
constexpr bool fits8(int nc, int nf) { return !(nc > 8 && nf > 3); }

// instances that plan() never picks (not compiled); at 4 waves the table is split again
// with the longer ring reach, so any 4-wave instance can occur. Far rows from the rotated
// rows (ROT) are picked for interpolated mode, 8 waves and at least one far entry only.
template <int MODE, int NC, int NF, int WAVES, bool ROT>
constexpr bool unused_instance() {
  return (WAVES == 8 && !fits8(NC, NF)) || (ROT && (MODE != 1 || WAVES != 8 || NF == 0));
}

template <int MODE, int NC, int NF, int WAVES, bool DEV, bool ROT>
hipError_t launch(const BqArgs& a, unsigned blocks, hipStream_t s) {
  if constexpr (unused_instance<MODE, NC, NF, WAVES, ROT>()) {
    return hipErrorInvalidValue;
  } else {
    const size_t smem = sizeof(BqSmem);
    static std::atomic<uint32_t> lds_set{0};
    hipError_t e = ensure_lds_limit(bwdq_ring_kernel<MODE, NC, NF, WAVES, DEV, ROT>, lds_set, (int)smem);
    if (e != hipSuccess) return e;
    bwdq_ring_kernel<MODE, NC, NF, WAVES, DEV, ROT><<<blocks, 64 * WAVES, smem, s>>>(a);
    return hipGetLastError();
  }
}

template <int MODE, int NC, int WAVES, bool DEV, bool ROT>
hipError_t launch_nf(const BqArgs& a, int n_far, unsigned blocks, hipStream_t s) {
  switch (n_far) {
    case 0: return launch<MODE, NC, 0, WAVES, DEV, false>(a, blocks, s);
    case 1: return launch<MODE, NC, 1, WAVES, DEV, ROT>(a, blocks, s);
    case 2: return launch<MODE, NC, 2, WAVES, DEV, ROT>(a, blocks, s);
    case 3: return launch<MODE, NC, 3, WAVES, DEV, ROT>(a, blocks, s);
    default: return launch<MODE, NC, 4, WAVES, DEV, ROT>(a, blocks, s);
  }
}

// kernel instance by (covered entries rounded up to 8 or 16, far entries, far rows rotated);
// with alpha in device memory (DEV) the counts are bounds over the alpha range
template <int MODE, int WAVES, bool DEV = false>
hipError_t launch_far(const BqArgs& a, int n_far, bool rot, unsigned blocks, hipStream_t s) {
  if (WAVES == 8 && rot) {
    return a.n_cov > 8 ? launch_nf<MODE, 16, WAVES, DEV, true>(a, n_far, blocks, s)
                       : launch_nf<MODE, 8, WAVES, DEV, true>(a, n_far, blocks, s);
  }
  return a.n_cov > 8 ? launch_nf<MODE, 16, WAVES, DEV, false>(a, n_far, blocks, s)
                     : launch_nf<MODE, 8, WAVES, DEV, false>(a, n_far, blocks, s);
}

// With alpha in device memory the counts are upper bounds over the alpha range.
int plan(const BwdArgs& f, int* n_cov, int* n_far) {
  auto split = [&](int waves) {
    if (f.plan != nullptr) {
      range_counts(f.alpha_lo, f.alpha_hi, f.base, f.n_base, f.W, f.mode, f.N, waves, n_cov, n_far);
    } else {
      split_table(f.tab, f.N, waves, n_cov, n_far);
    }
  };
  split(8);
  if (!fits8(*n_cov <= 8 ? 8 : 16, *n_far)) {
    split(4);
    return 4;
  }
  return 8;
}


}  // namespace

bool bwdq_ring_supported(const BwdArgs& f) {
  if (f.dtype != 1 || f.W > kMaxBand || f.N > (1LL << 30)) return false;
  int cov, far;
  plan(f, &cov, &far);
  return far <= kMaxFar && cov <= kMaxCov;
}

int bwdq_instance_key(const BwdArgs& f) {
  if (!bwdq_ring_supported(f)) return -1;
  int cov, far;
  const int waves = plan(f, &cov, &far);
  return waves * 1000 + (cov <= 8 ? 8 : 16) * 10 + far;
}

int64_t bwdq_ring_blocks(const BwdArgs& f) {
  int cov, far;
  const int kT = step_rows(plan(f, &cov, &far));
  const int64_t tiles = (f.N + kT - 1) / kT;
  return ring_segments(f.BH, tiles) * f.BH;
}

hipError_t launch_bwdq_ring(const BwdArgs& f, float* delta, float* part, uint32_t* ps, bf16_t* qr, bf16_t* kr) {
  BqArgs a;
  a.q = (const bf16_t*)f.q;
  a.k = (const bf16_t*)f.k;
  a.v = (const bf16_t*)f.v;
  a.o = (const bf16_t*)f.o;
  a.dout = (const bf16_t*)f.dout;
  a.lse = f.lse;
  a.dq = (bf16_t*)f.dq;
  a.delta = delta;
  a.dalpha_part = part;
  a.ps = ps;
  a.ps_slots = f.ps_slots;
  a.qr = qr;
  a.kr = kr;
  a.plan = f.plan;
  a.N = (int)f.N;
  a.W = f.W;
  int n_far;
  const int waves = plan(f, &a.n_cov, &n_far);
  for (int e = 0; e < kMaxCov; ++e) {
    a.dist[e] = e < a.n_cov ? f.tab.dist[e] : kMaxBand;
    a.w[e] = e < a.n_cov ? f.tab.w[e] : 0.f;
    a.f[e] = e < a.n_cov ? f.tab.f[e] : 0.f;
  }
  for (int x = 0; x < kMaxFar; ++x) {
    a.far_dist[x] = x < n_far ? f.tab.dist[a.n_cov + x] : 0;
    a.far_w[x] = x < n_far ? f.tab.w[a.n_cov + x] : 0.f;
    a.far_f[x] = x < n_far ? f.tab.f[a.n_cov + x] : 0.f;
  }
  int u = 0;
  for (int x = 0; x < n_far; ++x) {
    a.unc_dist[u++] = a.far_dist[x];
    if (f.mode == 1) a.unc_dist[u++] = a.far_dist[x] - 1;
  }
  for (; u < kMaxUnc; ++u) a.unc_dist[u] = 0;
  const int kT = step_rows(waves);
  int need = kMaxBand;
  for (int e = 0; e < a.n_cov; ++e) need = f.tab.dist[e] > need ? f.tab.dist[e] : need;
  a.warm = ((need + kT - 1) / kT) * kT;
  int early = kMaxBand;
  for (int e = 0; e < a.n_cov + n_far; ++e) early = f.tab.dist[e] > early ? f.tab.dist[e] : early;
  a.early_rows = early;
  const int64_t blocks = bwdq_ring_blocks(f);
  a.segs = (int)(blocks / f.BH);
  const int64_t tiles = (f.N + kT - 1) / kT;
  a.seg_len = (int)(((tiles + a.segs - 1) / a.segs) * kT);
  a.scale = (float)(1.0 / sqrt((double)kD));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kD));
  a.rope = f.rope;
  a.n_far = n_far;
  a.heads_per_plan = f.heads_per_plan;
  // Interpolated mode: far rows from the rotated rows when the rows before a segment that its
  // workgroup must rotate first (far reach minus the ring warm-up) are at most a quarter of
  // the segment.
  // With alpha in device memory the reach is bounded over the range: the largest usable
  // base entry's ceil(alpha_hi f) + 1 (the plan's far distances are alpha f rounded).
  int reach = 0;
  if (f.plan != nullptr) {
    for (int e = 0; e < f.n_base; ++e) {
      if ((double)f.alpha_lo * (double)f.base[e] >= (double)f.N) continue;
      const double d = ceil((double)f.alpha_hi * (double)f.base[e]) + 1.0;
      reach = (int)std::max<double>(reach, std::min<double>(d, (double)(f.N - 1)));
    }
  } else {
    for (int x = 0; x < n_far; ++x) reach = std::max(reach, a.far_dist[x]);
  }
  a.far_reach = reach;
  const bool rot = f.mode == 1 && waves == 8 && n_far > 0 && (int64_t)std::max(0, reach - a.warm) * 4 <= (int64_t)a.seg_len;
  if (f.plan != nullptr) {
    if (f.mode == 0) {
      return waves == 8 ? launch_far<0, 8, true>(a, n_far, rot, (unsigned)blocks, f.stream)
                        : launch_far<0, 4, true>(a, n_far, rot, (unsigned)blocks, f.stream);
    }
    return waves == 8 ? launch_far<1, 8, true>(a, n_far, rot, (unsigned)blocks, f.stream)
                      : launch_far<1, 4, true>(a, n_far, rot, (unsigned)blocks, f.stream);
  }
  if (f.mode == 0) {
    return waves == 8 ? launch_far<0, 8>(a, n_far, rot, (unsigned)blocks, f.stream)
                      : launch_far<0, 4>(a, n_far, rot, (unsigned)blocks, f.stream);
  }
  return waves == 8 ? launch_far<1, 8>(a, n_far, rot, (unsigned)blocks, f.stream)
                    : launch_far<1, 4>(a, n_far, rot, (unsigned)blocks, f.stream);
}

}  // namespace fib
