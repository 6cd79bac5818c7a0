// Key side of the backward pass on an LDS ring (bf16, D = 64, W <= 16, integer and
// interpolated offsets): dK and dV.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science summaries
// of arXiv 2606.28560, Method > Architecture and attention mechanism): key row j is read by
// the window queries j..j+W-1 and by query j + r for each table offset r. With
// P = exp(s - LSE_i), dP = <dO_i, V_j>, dS = P (dP - Delta_i) (Delta from the query side):
//   dK_j = R_j^T sum_i dS q^_i / sqrt(D),  dV_j = sum_i P dO_i
// (q^ the rotated query; R_j^T undoes the key's RoPE). Deterministic: each key's sums are
// formed by one lane group, no atomics.
//
// Design: the mirror image of the query side. Per step each wave takes 16 keys (rotated K^ and
// raw V in registers as MFMA B operands); the LDS ring holds the query rows ahead of them:
// rotated Q^ and dO, with LSE * log2(e) and Delta in each Q^ row's padding bytes. Logits
// S^T = Q^ K^T and dP^T = dO V^T on MFMA (window band: 32 queries x 16 keys; an offset: a
// 16-row query slab whose diagonal is used); dK^T = Q^T dS^T and dV^T = dO^T P^T on MFMA
// through transpose reads (addressed so that lane (n, g) accumulates dims 8g..8g+7 and
// 32+8g..32+8g+7 of key n). The ring leads the keys by the largest covered offset: at step
// p0 it receives the query rows p0 + kLead ... Offsets beyond the ring read q and dO rows
// from global memory. Integer offsets: raw q rows, rotated here (relative RoPE <R_r q_i, k_j>,
// their dK terms added after R_j is undone). Interpolated offsets, where this kernel's VALU
// work bounds it: the rotated rows K^ and Q^ come from the workspace, where the query side
// (the kernel before this one) wrote every row, and a far entry's dK terms dS q^ join the
// rotated frame before R_j is undone.
//
// Interpolated offsets: key j is the lower row (weight 1 - w) of query j + c and the upper
// row (weight w) of query j + c - 1, for each entry (c = ceil(d), w = c - d). The query side
// has stored each (query, entry)'s P and dS (ps_pack), so no logit of an entry is
// recomputed here: the two query slabs j0 + c + n and j0 + c - 1 + n pair up in one MFMA per
// output block with the diagonal weights ((1 - w) dS_lo, w dS_hi) and ((1 - w) P_lo, w P_hi).
// A far entry's upper query row of key n is the lower row of key n - 1: each lane loads one
// row, takes its neighbour's with a DPP row shift, and the one row that no lane of the wave
// holds (j0 + c - 1, for key j0) is loaded spread over the wave, one dword per lane.
#include "ring_common.h"

namespace fib {
namespace {

using namespace ring;

struct BkArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dout;
  const float* lse;
  const float* delta;
  const uint32_t* ps;  // interpolated: (P, dS) per (query, entry), [head][ps_slots][N]
  int ps_slots;
  const bf16_t* qr;    // interpolated: rotated rows R_i q_i, [head][N][D] (from the query side)
  const bf16_t* kr;    // interpolated: rotated rows R_j k_j, [head][N][D] (from the query side)
  bf16_t* dk;
  bf16_t* dv;
  int N;
  int W;
  int n_cov;
  int seg_len;
  int segs;
  int lead;  // ring lead: query rows [p0, p0 + lead) are in the ring before step p0 inserts
  float scale;
  float scale_log2;
  int dist[kMaxCov];
  float w[kMaxCov];
  int far_dist[kMaxFar];
  float far_w[kMaxFar];
  Rope rope;
  const DevPlan* plan;  // alpha in device memory: the split above comes from here (DEV instances)
  int n_far;            // far entries in use (DEV instances: NF is an upper bound)
  int heads_per_plan;   // DEV instances: head h reads plan[h / heads_per_plan]
  // d(alpha) per layer, formed here because this kernel runs after the query side: block b <
  // dal_layers writes dal_out[b] = the ordered sum of the dal_n partials of layer b
  // (interpolated mode) or 0 (integer mode); dal_out may be null
  const float* dal_part;
  int64_t dal_n;
  float* dal_out;
  int dal_layers;
};

struct __align__(16) BkSmem {
  uint8_t ringQ[(kP + kMirror) * kRow];  // Q^ rows; bytes 128..135: (LSE * log2 e, Delta)
  uint8_t ringD[(kP + kMirror) * kRow];  // dO rows
  float2 unc_cs[kMaxUnc][kHalf];  // integer mode: the far offsets' rotations
  float2 base_cs[2][2][kHalf];    // [buffer][keys, queries (integer mode)]
  float2 warm_cs[8][kHalf];       // integer mode: the warm-up query rows' rotations
};

// Q^ (rotated) and dO rows of the far queries j0 + r + n (row N - 1 past the end; masked), and their
// LSE and Delta as loaded (the use masks the rows past the end: a select here, next to the
// load, would make the wave wait for the load at once)
template <int NF>
struct FarQ {
  uint4 q[NF > 0 ? NF : 1][2];
  uint4 d[NF > 0 ? NF : 1][2];
  float lse2[NF > 0 ? NF : 1];
  float dlt[NF > 0 ? NF : 1];
};

// n_use: far slots in use (NF, or fewer in DEV instances: the unused slots get zero rows and
// an infinite LSE, i.e. weight 0, without a load; n_use is wave-uniform)
template <int NF>
__device__ __forceinline__ void load_far_q(const int* fdist, int n_use, FarQ<NF>& fq, const BkArgs& a,
                                           const bf16_t* Qh, const bf16_t* Dh, const float* Lh, const float* Th, int j0,
                                           int n, int g, int lane_off) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f >= n_use) {
      fq.q[f][0] = fq.q[f][1] = fq.d[f][0] = fq.d[f][1] = make_uint4(0, 0, 0, 0);
      fq.lse2[f] = INFINITY;
      fq.dlt[f] = 0.f;
      continue;
    }
    const int r0 = j0 + fdist[f];
    int64_t off;
    int r = r0 + n;
    if (r0 + 15 < a.N) {
      off = (int64_t)r0 * kD + lane_off;
    } else {
      off = (int64_t)(r < a.N ? r : a.N - 1) * kD + 8 * g;
    }
    fq.q[f][0] = *reinterpret_cast<const uint4*>(Qh + off);
    fq.q[f][1] = *reinterpret_cast<const uint4*>(Qh + off + kHalf);
    fq.d[f][0] = *reinterpret_cast<const uint4*>(Dh + off);
    fq.d[f][1] = *reinterpret_cast<const uint4*>(Dh + off + kHalf);
    const int rc = r < a.N ? r : a.N - 1;
    fq.lse2[f] = Lh[rc];
    fq.dlt[f] = Th[rc];
  }
}

// Interpolated far entries, per entry: the lower query row j0 + c + n of the lane's key (Q^
// and dO, the lane's dims), the row j0 + c - 1 spread over the wave (lane l: dword l & 31
// of Q^ if l < 32, else of dO) and the stored (P, dS) of the key's lower and upper query.
template <int NF>
struct FarQI {
  uint4 q[NF > 0 ? NF : 1][2];
  uint4 d[NF > 0 ? NF : 1][2];
  uint32_t ex[NF > 0 ? NF : 1];
  uint32_t pl[NF > 0 ? NF : 1];  // as loaded: rows past the end are masked at the use
  uint32_t ph[NF > 0 ? NF : 1];
};

// loads at a wave-uniform base plus a small per-lane byte offset (the base stays in scalar
// registers; only the 32-bit offset is per lane)
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
}
__device__ __forceinline__ uint32_t ld4(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(base) + off);
}

template <int NF>
__device__ __forceinline__ void load_far_qi(const int* fdist, int n_use, FarQI<NF>& fq, const BkArgs& a,
                                            const bf16_t* Qh, const bf16_t* Dh, const uint32_t* Sh, int n_cov, int j0,
                                            int l, int n, int g) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f >= n_use) {  // (as in load_far_q: (P, dS) = 0 gives the slot weight 0)
      fq.q[f][0] = fq.q[f][1] = fq.d[f][0] = fq.d[f][1] = make_uint4(0, 0, 0, 0);
      fq.ex[f] = fq.pl[f] = fq.ph[f] = 0u;
      continue;
    }
    const int r0 = j0 + fdist[f];
    // rows past the end repeat row N - 1 (their weights are zero)
    const int rb = r0 < a.N ? r0 : a.N - 1;
    const int r = r0 + n;
    const uint32_t off = (uint32_t)(((r < a.N ? r : a.N - 1) - rb) * kD + 8 * g) * 2u;
    const bf16_t* qb = Qh + (int64_t)rb * kD;
    const bf16_t* db = Dh + (int64_t)rb * kD;
    fq.q[f][0] = ld16(qb, off);
    fq.q[f][1] = ld16(qb, off + 2 * kHalf);
    fq.d[f][0] = ld16(db, off);
    fq.d[f][1] = ld16(db, off + 2 * kHalf);
    // (every load is in bounds; the words of rows past the end are masked where they are
    // used, so no select waits on a load here)
    const int re = r0 - 1 < a.N ? r0 - 1 : a.N - 1;
    fq.ex[f] = ld4((l < 32 ? Qh : Dh) + (int64_t)re * kD, 4u * (uint32_t)(l & 31));
    const uint32_t* se = Sh + (size_t)(n_cov + f) * a.N + rb;
    fq.pl[f] = ld4(se, (uint32_t)((r < a.N ? r : a.N - 1) - rb) * 4u);
    fq.ph[f] = ld4(se - 1, (uint32_t)((r - 1 < a.N ? r - 1 : a.N - 1) - rb + 1) * 4u);
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

template <int MODE, int NC, int NF, bool DEV>
__global__ __launch_bounds__(512, 1) void bwdk_ring_kernel(BkArgs a) {
  constexpr int WAVES = 8;
  constexpr int kThreads = 64 * WAVES;
  constexpr int kT = step_rows(WAVES);
  extern __shared__ __align__(16) uint8_t smem_raw[];
  BkSmem& sm = *reinterpret_cast<BkSmem*>(smem_raw);
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
    lcl = pl->s8;
  }
  const int S_n_cov = DEV ? lcl.n_cov : a.n_cov;
  const int S_n_far = DEV ? lcl.n_far : a.n_far;
  const int S_lead = DEV ? ((lcl.need + kT - 1) / kT) * kT : a.lead;
  auto S_dist = [&](int x) -> int { if constexpr (DEV) return lcl.dist[x]; else return a.dist[x]; };
  auto S_w = [&](int x) -> float { if constexpr (DEV) return lcl.w[x]; else return a.w[x]; };
  auto S_far_dist = [&](int x) -> int { if constexpr (DEV) return lcl.far_dist[x]; else return a.far_dist[x]; };
  auto S_far_w = [&](int x) -> float { if constexpr (DEV) return lcl.far_w[x]; else return a.far_w[x]; };


  if constexpr (MODE == 0) {
    for (int x = tid; x < NF * kHalf; x += kThreads) {
      const int u = x / kHalf, j = x % kHalf;
      int d;
      if constexpr (DEV) d = pl->s8.far_dist[u];
      else d = S_far_dist(u);  // (a's arrays: constant indices in DEV instances)
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
  // registers through the loop: the window masks (query row 4g + v of slab 0, 16 + 4g + v of
  // slab 1, reads key n when 0 <= row - n < W) and the selectors of diag_block. (The empty asm
  // makes W opaque, so the compiler does not hoist them out of the loop.) Masks select -inf
  // instead of adding it, so a NaN logit outside the attended set stays masked.
  auto window_in = [&](bool* in0, bool* in1) {
    int Wp = a.W;
    asm volatile("" : "+s"(Wp));
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int d0 = 4 * g + v - n, d1 = 16 + 4 * g + v - n;
      in0[v] = d0 >= 0 && d0 < Wp;
      in1[v] = d1 < Wp;
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
  // transpose reads: lane (jr, jc) of group g reads row 4g + jr at dims 8 jc + 4 h + 32 h2
  // (output block mb = 2 h2 + h): output row 4g' + v of block mb is dim 8g' + 4h + 32h2 + v
  const int lane_t = (4 * g + jr) * kRow + 16 * jc;
  // the lane's (LSE, Delta) pair of slab row 4g + v is at row_off + lane_lv + v * kRow
  const int lane_lv = 4 * g * kRow + 128;
  const int lane_off = n * kD + 8 * g;

  const int64_t head = blockIdx.x / a.segs;
  const int seg = blockIdx.x % a.segs;
  const int s0 = seg * a.seg_len;
  const int s1 = s0 + a.seg_len < N ? s0 + a.seg_len : N;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const bf16_t* Vh = a.v + hoff;
  const bf16_t* Dh = a.dout + hoff;
  const float* Lh = a.lse + (size_t)head * N;
  const float* Th = a.delta + (size_t)head * N;
  const uint32_t* Sh = MODE == 1 ? a.ps + (size_t)head * a.ps_slots * N : nullptr;
  // integer mode: raw q and k rows, rotated here; interpolated: the rotated rows
  const bf16_t* Qs = MODE == 1 ? a.qr + hoff : a.q + hoff;
  const bf16_t* Ks = MODE == 1 ? a.kr + hoff : a.k + hoff;

  auto row_elems = [&](int rb) -> int64_t {
    if (rb + 15 < N) return (int64_t)rb * kD + lane_off;
    const int r = rb + n < N ? rb + n : N - 1;
    return (int64_t)r * kD + 8 * g;
  };
  auto load2 = [&](const bf16_t* base, int64_t off, uint4* x) {
    x[0] = *reinterpret_cast<const uint4*>(base + off);
    x[1] = *reinterpret_cast<const uint4*>(base + off + kHalf);
  };
  // query row qb + n into the ring: Q^ (integer mode: rotated here by cs; interpolated: as
  // the query side wrote it), dO, (LSE log2e, Delta); rows past the end hold zeros and
  // LSE = +inf (P = 0)
  auto put_query = [&](int qb, const float2* cs, const uint4* q2, const uint4* d2, float lse, float dlt) {
    const bool live = qb + n < N;
    const uint4 z = make_uint4(0, 0, 0, 0);
    uint4 r0 = q2[0], r1 = q2[1];
    if constexpr (MODE == 0) {
      float qf[16];
      unpack8(q2[0], qf);
      unpack8(q2[1], qf + 8);
      rotate_pack_f(qf, cs, &r0, &r1);
    }
    if (!live) r0 = r1 = z;
    const uint4 d0 = live ? d2[0] : z, d1 = live ? d2[1] : z;
    const float2 ld = live ? make_float2(lse * log2e, dlt) : make_float2(INFINITY, 0.f);
    const int slot = qb & (kP - 1);
    auto put = [&](int ro) {
      lds_write16(sm.ringQ + ro + 16 * g, 0, r0);
      lds_write16(sm.ringQ + ro + 16 * g, 64, r1);
      lds_write16(sm.ringD + ro + 16 * g, 0, d0);
      lds_write16(sm.ringD + ro + 16 * g, 64, d1);
      if (g == 0) *reinterpret_cast<float2*>(sm.ringQ + ro + 128) = ld;
    };
    put((slot + n) * kRow);
    if (slot < kMirror) put((slot + kP + n) * kRow);
  };
  auto compose = [&](float2 b, float2 t) {
    return make_float2(b.x * t.x - b.y * t.y, b.y * t.x + b.x * t.y);
  };

  // ---- warm-up: query rows [s0, s0 + lead) (lead is a step multiple)
  const int n_warm = S_lead / kT;
  if (tid < kHalf * (MODE == 0 ? n_warm + 2 : 1)) {
    const int j = tid / kHalf, t = tid % kHalf;
    if (MODE == 1 || j == n_warm) sm.base_cs[0][0][t] = rope_cs(s0, a.rope.rev[t]);
    else if (j < n_warm) sm.warm_cs[j][t] = rope_cs(s0 + j * kT, a.rope.rev[t]);
    else sm.base_cs[0][1][t] = rope_cs(s0 + S_lead, a.rope.rev[t]);
  }
  // this step's keys and inserted query rows, prefetched one step ahead
  uint4 pk[2], pv[2], pq[2], pd[2];
  float plse, pdlt;
  // interpolated: the stored (P, dS) of the covered entries' lower and upper query of the
  // lane's key, as loaded (only the diagonal lane's words of entries in use and of rows
  // before the end count: the use masks the others)
  uint32_t psl[MODE == 1 ? NC : 1], psh[MODE == 1 ? NC : 1];
  auto load_ps = [&](int pb) {
    if constexpr (MODE == 1) {
      // (loads at clamped rows; the words that must not count are masked where they are
      // used, so no select waits on a load here)
      const int jb = pb + 16 * wave;
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        const int b = jb + S_dist(e) - 1 < N ? jb + S_dist(e) - 1 : N - 1;  // >= 0
        const int ilo = jb + S_dist(e) + n;
        // slots past the covered entries read entry 0's words (in bounds: the head has
        // a.ps_slots >= 1 entry rows; the values are selected away below)
        const uint32_t* se = Sh + (size_t)(e < S_n_cov ? e : 0) * N + b;
        psl[e] = ld4(se, (uint32_t)((ilo < N ? ilo : N - 1) - b) * 4u);
        psh[e] = ld4(se, (uint32_t)((ilo - 1 < N ? ilo - 1 : N - 1) - b) * 4u);
      }
    }
  };
  auto load_step = [&](int pb) {
    const int64_t ko = row_elems(pb + 16 * wave);
    load2(Ks, ko, pk);
    load2(Vh, ko, pv);
    const int qb = pb + S_lead + 16 * wave;
    const int64_t qo = row_elems(qb);
    load2(Qs, qo, pq);
    load2(Dh, qo, pd);
    const int r = qb + n < N ? qb + n : N - 1;
    plse = Lh[r];
    pdlt = Th[r];
  };
  load_step(s0);
  load_ps(s0);
  __syncthreads();
  {
    // kWB steps of warm rows in flight at once, then (integer mode: rotated and) stored
    constexpr int kWB = 3;
    for (int j0 = 0; j0 < n_warm; j0 += kWB) {
      uint4 wq[kWB][2], wd[kWB][2];
      float wl[kWB], wt[kWB];
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          const int qb = s0 + (j0 + jj) * kT + 16 * wave;
          load2(Qs, row_elems(qb), wq[jj]);
          load2(Dh, row_elems(qb), wd[jj]);
          const int r = qb + n < N ? qb + n : N - 1;
          wl[jj] = Lh[r];
          wt[jj] = Th[r];
        }
      }
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          const int qb = s0 + (j0 + jj) * kT + 16 * wave;
          float2 cs[8];
          if constexpr (MODE == 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) cs[t] = compose(sm.warm_cs[j0 + jj][8 * g + t], cs_t[t]);
          }
          put_query(qb, cs, wq[jj], wd[jj], wl[jj], wt[jj]);
        }
      }
    }
  }
  FarQ<MODE == 0 ? NF : 0> fq;
  FarQI<MODE == 1 ? NF : 0> fi;
  if constexpr (MODE == 0)
    load_far_q<NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fq, a, Qs, Dh, Lh, Th, s0 + 16 * wave, n, g, lane_off);
  else
    load_far_qi<NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fi, a, Qs, Dh, Sh, S_n_cov, s0 + 16 * wave, l, n, g);

  int buf = 0;
  for (int p0 = s0; p0 < s1; p0 += kT, buf ^= 1) {
    // ---- this step's keys (rotated K^ and raw V; integer mode: raw K for the far offsets)
    // and the query rows entering the ring
    uint4 kh0 = pk[0], kh1 = pk[1];
    const uint4 kraw0 = pk[0], kraw1 = pk[1], v0 = pv[0], v1 = pv[1];
    if constexpr (MODE == 0) {
      float2 csk[8], csq[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        csk[t] = compose(sm.base_cs[buf][0][8 * g + t], cs_t[t]);
        csq[t] = compose(sm.base_cs[buf][1][8 * g + t], cs_t[t]);
      }
      float kf[16];
      unpack8(pk[0], kf);
      unpack8(pk[1], kf + 8);
      rotate_pack_f(kf, csk, &kh0, &kh1);
      put_query(p0 + S_lead + 16 * wave, csq, pq, pd, plse, pdlt);
    } else {
      put_query(p0 + S_lead + 16 * wave, nullptr, pq, pd, plse, pdlt);
    }
    __syncthreads();
    const int pn = p0 + kT;
    // (the next step's keys and query rows are requested after the covered entries, so that
    // their registers are not held through the step's register peak: held, they cost spills
    // whose reloads wait for every load in flight)
    if (wave == 0 && l < kHalf) {
      sm.base_cs[buf ^ 1][0][l] = rope_cs(pn, rev_l);
      if constexpr (MODE == 0) sm.base_cs[buf ^ 1][1][l] = rope_cs(pn + S_lead, rev_l);
    }

    const int j0 = p0 + 16 * wave;
    const int jk = j0 + n;  // this lane's key
    const bf16x8 bk0 = as_bf8(kh0), bk1 = as_bf8(kh1);
    const bf16x8 bv0 = as_bf8(v0), bv1 = as_bf8(v1);
    f4 acck[4], accv[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acck[mb] = accv[mb] = f4{0, 0, 0, 0};

    // ---- window band: query rows j0 + kappa, kappa < 32
    const int band = row_off(j0);
    uint32_t sel[4];
    diag_sel(sel);
    {
      f4 S0 = {0, 0, 0, 0}, S1 = {0, 0, 0, 0}, D0 = {0, 0, 0, 0}, D1 = {0, 0, 0, 0};
      const int sa = band + lane_k;
      S0 = mfma32(as_bf8(lds_read16(sm.ringQ, sa)), bk0, S0);
      S0 = mfma32(as_bf8(lds_read16(sm.ringQ, sa + 64)), bk1, S0);
      S1 = mfma32(as_bf8(lds_read16(sm.ringQ, sa + 16 * kRow)), bk0, S1);
      S1 = mfma32(as_bf8(lds_read16(sm.ringQ, sa + 16 * kRow + 64)), bk1, S1);
      D0 = mfma32(as_bf8(lds_read16(sm.ringD, sa)), bv0, D0);
      D0 = mfma32(as_bf8(lds_read16(sm.ringD, sa + 64)), bv1, D0);
      D1 = mfma32(as_bf8(lds_read16(sm.ringD, sa + 16 * kRow)), bv0, D1);
      D1 = mfma32(as_bf8(lds_read16(sm.ringD, sa + 16 * kRow + 64)), bv1, D1);
      float p[8], ds[8];
      bool in0[4], in1[4];
      window_in(in0, in1);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float2 l0 = *reinterpret_cast<const float2*>(sm.ringQ + band + lane_lv + v * kRow);
        const float2 l1 = *reinterpret_cast<const float2*>(sm.ringQ + band + lane_lv + (16 + v) * kRow);
        p[v] = ex2((in0[v] ? S0[v] * sl2 : -INFINITY) - l0.x);
        p[4 + v] = ex2((in1[v] ? S1[v] * sl2 : -INFINITY) - l1.x);
        ds[v] = p[v] * (D0[v] - l0.y);
        ds[4 + v] = p[4 + v] * (D1[v] - l1.y);
      }
      const bf16x8 bp = __builtin_bit_cast(
          bf16x8, make_uint4(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]), pack_bf2(p[4], p[5]), pack_bf2(p[6], p[7])));
      // dS as bf16 plus its rounding residual (a second MFMA): the window's dS (whose
      // weights P reach 1 near the sequence start) are not rounded to 8 significant bits
      uint32_t hs[4], ls[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        hs[x] = pack_bf2(ds[2 * x], ds[2 * x + 1]);
        ls[x] = pack_bf2(ds[2 * x] - bf_lo(hs[x]), ds[2 * x + 1] - bf_hi(hs[x]));
      }
      const bf16x8 bs = __builtin_bit_cast(bf16x8, make_uint4(hs[0], hs[1], hs[2], hs[3]));
      const bf16x8 bs2 = __builtin_bit_cast(bf16x8, make_uint4(ls[0], ls[1], ls[2], ls[3]));
      const int r0 = band + lane_t, r1 = r0 + 16 * kRow;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int o = 8 * (mb & 1) + 64 * (mb >> 1);
        const bf16x8 aq = cat_bf8(tr16(sm.ringQ, r0 + o), tr16(sm.ringQ, r1 + o));
        acck[mb] = mfma32(aq, bs, acck[mb]);
        acck[mb] = mfma32(aq, bs2, acck[mb]);
        accv[mb] = mfma32(cat_bf8(tr16(sm.ringD, r0 + o), tr16(sm.ringD, r1 + o)), bp, accv[mb]);
      }
    }
    // ---- covered offsets: query slab rows j0 + r + n (diagonal), two offsets per MFMA
    if constexpr (MODE == 0) {
#pragma unroll
    for (int e = 0; e < NC; e += 2) {
      float p2[2], ds2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sl = row_off(j0 + S_dist(e + h));
        f4 S = {0, 0, 0, 0}, P = {0, 0, 0, 0};
        S = mfma32(as_bf8(lds_read16(sm.ringQ, sl + lane_k)), bk0, S);
        S = mfma32(as_bf8(lds_read16(sm.ringQ, sl + lane_k + 64)), bk1, S);
        P = mfma32(as_bf8(lds_read16(sm.ringD, sl + lane_k)), bv0, P);
        P = mfma32(as_bf8(lds_read16(sm.ringD, sl + lane_k + 64)), bv1, P);
        // (LSE, Delta) of query row j0 + r + n
        const float2 ld = *reinterpret_cast<const float2*>(sm.ringQ + sl + n * kRow + 128);
        float x = diag_lane ? sel4(S, l) * sl2 : -INFINITY;
        if (e + h >= S_n_cov) x = -INFINITY;
        p2[h] = ex2(x - ld.x);
        ds2[h] = p2[h] * (sel4(P, l) - ld.y);
      }
      const bf16x8 bp = diag_block(pack_bf2(p2[0], p2[1]), sel);
      const bf16x8 bs = diag_block(pack_bf2(ds2[0], ds2[1]), sel);
      const int ra = row_off(j0 + S_dist(e)) + lane_t, rb = row_off(j0 + S_dist(e + 1)) + lane_t;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int o = 8 * (mb & 1) + 64 * (mb >> 1);
        acck[mb] = mfma32(cat_bf8(tr16(sm.ringQ, ra + o), tr16(sm.ringQ, rb + o)), bs, acck[mb]);
        accv[mb] = mfma32(cat_bf8(tr16(sm.ringD, ra + o), tr16(sm.ringD, rb + o)), bp, accv[mb]);
      }
    }
    } else {
      // interpolated: the lower query slab j0 + c + n and the upper one j0 + c - 1 + n of an
      // entry in one MFMA, with the stored P and dS (entries past n_cov have zero weights).
      // The weighted dS ((1 - w) dS_lo, w dS_hi) enter as a bf16 pair plus the pair of their
      // rounding residuals (two MFMAs): the weights keep the stored dS's 12 significant bits.
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        const float w = S_w(e);
        const int ilo = jk + S_dist(e);  // the key's lower query
        const bool use = diag_lane && e < S_n_cov;
        const uint32_t wl = use && ilo < N ? psl[e] : 0u, wh = use && ilo - 1 < N ? psh[e] : 0u;
        const float xs = ps_ds(wl) * (1.f - w), ys = ps_ds(wh) * w;
        const uint32_t hs = pack_bf2(xs, ys);
        const bf16x8 bs = diag_block(hs, sel);
        const bf16x8 bs2 = diag_block(pack_bf2(xs - bf_lo(hs), ys - bf_hi(hs)), sel);
        const bf16x8 bp = diag_block(pack_bf2(ps_p(wl) * (1.f - w), ps_p(wh) * w), sel);
        const int ra = row_off(j0 + S_dist(e)) + lane_t, rb = row_off(j0 + S_dist(e) - 1) + lane_t;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int o = 8 * (mb & 1) + 64 * (mb >> 1);
          const bf16x8 aq = cat_bf8(tr16(sm.ringQ, ra + o), tr16(sm.ringQ, rb + o));
          acck[mb] = mfma32(aq, bs, acck[mb]);
          acck[mb] = mfma32(aq, bs2, acck[mb]);
          accv[mb] = mfma32(cat_bf8(tr16(sm.ringD, ra + o), tr16(sm.ringD, rb + o)), bp, accv[mb]);
        }
      }
    }
    load_step(pn < s1 ? pn : p0);
    // ---- interpolated far offsets: Q^ and dO rows from global memory; dK^ and dV terms on
    // VALU with the stored weights of the query, added in the rotated frame before R_j is
    // undone below
    if constexpr (MODE == 1) {
      // the lower query row (the lane's) and the upper row, both Q^, weighted by the stored dS
      // in fp32; the dO rows weighted by the stored P in bf16, as on the ring path.
      // (Scheduling barriers keep each entry's cross-lane moves and unpacked values from
      // spreading over the other entries and the MFMA part, where they would hold registers;
      // the first one also keeps work of this section out of the window band, where it would
      // wait for the far rows.)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const float w = S_far_w(f);
        // (a slot beyond the table weighs nothing)
        const float keep = DEV && f >= S_n_far ? 0.f : 1.f;
        const int rq = jk + S_far_dist(f);  // the key's lower far query (rows past the end count 0)
        const uint32_t wl = rq < N ? fi.pl[f] : 0u, wh = rq - 1 < N ? fi.ph[f] : 0u;
        const float al = keep * ps_ds(wl) * (1.f - w), ah = keep * ps_ds(wh) * w;
        const uint32_t pw = pack_bf2(keep * ps_p(wl) * (1.f - w), keep * ps_p(wh) * w);
#pragma unroll
        for (int tsr = 0; tsr < 2; ++tsr) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // words 2hh, 2hh + 1 of each 16-byte half of the lane's slice: dims 8g + 4hh..+3 and
          // 32 + 8g + 4hh..+3
          const uint4 a0 = tsr == 0 ? fi.q[f][0] : fi.d[f][0], a1 = tsr == 0 ? fi.q[f][1] : fi.d[f][1];
          uint32_t lo[4] = {hh == 0 ? a0.x : a0.z, hh == 0 ? a0.y : a0.w, hh == 0 ? a1.x : a1.z, hh == 0 ? a1.y : a1.w};
          uint32_t ex = fi.ex[f];
          // (empty asm: pins the uses of these registers below this point)
#pragma unroll
          for (int x = 0; x < 4; ++x) asm volatile("" : "+v"(lo[x]));
          asm volatile("" : "+v"(ex));
          uint32_t hi[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            // the same word of row j0 + c - 1 (tensor tsr, 16-byte half x / 2, word 2hh + x % 2),
            // for the lanes of key 0; every other lane takes lane n - 1's row
            const int src = 32 * tsr + 16 * (x >> 1) + 4 * g + 2 * hh + (x & 1);
            const int e = __builtin_amdgcn_ds_bpermute(4 * src, (int)ex);
            hi[x] = (uint32_t)__builtin_amdgcn_update_dpp(e, (int)lo[x], 0x111, 0xf, 0xf, false);
          }
          // lo[x], hi[x]: word x of the lower and the upper row; dim 8g + 4hh + t is half t % 2 of
          // word t / 2 (accumulator element acc[hh][t]), dim 32 + 8g + 4hh + t the same half of
          // word 2 + t / 2 (element acc[2 + hh][t])
          if (tsr == 0) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t xa = lo[t >> 1], xb = lo[2 + (t >> 1)], ya = hi[t >> 1], yb = hi[2 + (t >> 1)];
              const float la = (t & 1) ? bf_hi(xa) : bf_lo(xa), lb = (t & 1) ? bf_hi(xb) : bf_lo(xb);
              const float ua = (t & 1) ? bf_hi(ya) : bf_lo(ya), ub = (t & 1) ? bf_hi(yb) : bf_lo(yb);
              acck[hh][t] = fmaf(al, la, fmaf(ah, ua, acck[hh][t]));
              acck[2 + hh][t] = fmaf(al, lb, fmaf(ah, ub, acck[2 + hh][t]));
            }
          } else {
            // dO: (lower, upper) pairs of each dim against the bf16 weights (P_lo, P_hi)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
              accv[hh][t] = dot2(__builtin_amdgcn_perm(hi[t >> 1], lo[t >> 1], sel), pw, accv[hh][t]);
              accv[2 + hh][t] = dot2(__builtin_amdgcn_perm(hi[2 + (t >> 1)], lo[2 + (t >> 1)], sel), pw,
                                     accv[2 + hh][t]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        }
      }
    }
    // undo R_j on dK^: dims 8g+t (acck[0], acck[1]) pair with 32+8g+t (acck[2], acck[3])
    float kl[8], khv[8], vl[8], vhv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // the key's rotation, recomputed (base_cs[buf] stays valid through the step)
      const float2 c = compose(sm.base_cs[buf][0][8 * g + t], cs_t[t]);
      const float x = acck[t >> 2][t & 3], y = acck[2 + (t >> 2)][t & 3];
      kl[t] = x * c.x + y * c.y;
      khv[t] = y * c.x - x * c.y;
      vl[t] = accv[t >> 2][t & 3];
      vhv[t] = accv[2 + (t >> 2)][t & 3];
    }

    // ---- integer far offsets: raw q (rotated by R_r, bf16) and dO rows from global memory;
    // dK and dV terms on VALU with the bf16 weights (dS, P) of the query's diagonal lane, in
    // the un-rotated frame. (Scheduling barrier: the far rows, requested at the end of the
    // previous step, are first waited for here, not in the window band, where work hoisted
    // from this section would wait for them)
    if constexpr (MODE == 0) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      uint4 r0, r1;
      {
        float qf[16];
        unpack8(fq.q[f][0], qf);
        unpack8(fq.q[f][1], qf + 8);
        rotate_pack_f(qf, &sm.unc_cs[f][8 * g], &r0, &r1);
      }
      f4 S = {0, 0, 0, 0};
      S = mfma32(as_bf8(r0), as_bf8(kraw0), S);
      S = mfma32(as_bf8(r1), as_bf8(kraw1), S);
      const int rq = jk + S_far_dist(f);  // the key's far query
      const float lse2 = rq < N ? fq.lse2[f] * log2e : INFINITY;
      float x = (diag_lane ? sel4(S, l) * sl2 : -INFINITY) - lse2;
      if (DEV && f >= S_n_far) x = -INFINITY;  // slot beyond the table
      const float p = __uint_as_float((uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)__float_as_uint(ex2(x))));
      const float dp = quad_add(dot16_bf(fq.d[f][0], fq.d[f][1], v0, v1));
      const uint32_t y = pack_bf2(p * (dp - fq.dlt[f]), p);  // (dS, P) in bf16
      const uint32_t s_lo = y & 0xffffu, s_hi = y << 16, p_lo = y >> 16, p_hi = y & 0xffff0000u;
      const uint32_t qe[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      const uint32_t de[8] = {fq.d[f][0].x, fq.d[f][0].y, fq.d[f][0].z, fq.d[f][0].w,
                              fq.d[f][1].x, fq.d[f][1].y, fq.d[f][1].z, fq.d[f][1].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kl[2 * u] = dot2(qe[u], s_lo, kl[2 * u]);
        kl[2 * u + 1] = dot2(qe[u], s_hi, kl[2 * u + 1]);
        khv[2 * u] = dot2(qe[4 + u], s_lo, khv[2 * u]);
        khv[2 * u + 1] = dot2(qe[4 + u], s_hi, khv[2 * u + 1]);
        vl[2 * u] = dot2(de[u], p_lo, vl[2 * u]);
        vl[2 * u + 1] = dot2(de[u], p_hi, vl[2 * u + 1]);
        vhv[2 * u] = dot2(de[4 + u], p_lo, vhv[2 * u]);
        vhv[2 * u + 1] = dot2(de[4 + u], p_hi, vhv[2 * u + 1]);
      }
    }
    }

    // ---- epilogue: dK = scale * (the lane's dims), dV
    // interpolated: the next step's (P, dS), requested after the far terms (which is where the
    // registers run short); they are first used after the next step's window band
    load_ps(pn < s1 ? pn : p0);
    if constexpr (MODE == 1) {
      // (empty asm: the sums are formed here, not sunk into the conditional store below
      // past the loads that follow it)
#pragma unroll
      for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(kl[t]), "+v"(khv[t]), "+v"(vl[t]), "+v"(vhv[t]));
    }
    if (jk < s1) {
      // (wave-uniform row bases plus the lane's 32-bit byte offset, made opaque here so that
      // the compiler does not form per-lane 64-bit addresses before the loop and hold them
      // through it)
      char* kp = reinterpret_cast<char*>(a.dk + hoff + (int64_t)j0 * kD);
      char* vp = reinterpret_cast<char*>(a.dv + hoff + (int64_t)j0 * kD);
      uint32_t lb = 2u * (uint32_t)lane_off;
      asm volatile("" : "+v"(lb));
      uint4 x0, x1, y0, y1;
      x0.x = pack_bf2(kl[0] * a.scale, kl[1] * a.scale);
      x0.y = pack_bf2(kl[2] * a.scale, kl[3] * a.scale);
      x0.z = pack_bf2(kl[4] * a.scale, kl[5] * a.scale);
      x0.w = pack_bf2(kl[6] * a.scale, kl[7] * a.scale);
      x1.x = pack_bf2(khv[0] * a.scale, khv[1] * a.scale);
      x1.y = pack_bf2(khv[2] * a.scale, khv[3] * a.scale);
      x1.z = pack_bf2(khv[4] * a.scale, khv[5] * a.scale);
      x1.w = pack_bf2(khv[6] * a.scale, khv[7] * a.scale);
      y0 = pack8(vl);
      y1 = pack8(vhv);
      *reinterpret_cast<uint4*>(kp + lb) = x0;
      *reinterpret_cast<uint4*>(kp + lb + 2 * kHalf) = x1;
      *reinterpret_cast<uint4*>(vp + lb) = y0;
      *reinterpret_cast<uint4*>(vp + lb + 2 * kHalf) = y1;
    }
    // the next step's far rows, requested after the stores: the far terms above feed only the
    // stores, so requested earlier the new rows would be held alongside them (and, before the
    // conditional store, they need copies at the end of the step that wait for every load)
    if constexpr (MODE == 0)
      load_far_q<NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fq, a, Qs, Dh, Lh, Th, j0 + kT, n, g, lane_off);
    if constexpr (MODE == 1) load_far_qi<NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fi, a, Qs, Dh, Sh, S_n_cov, j0 + kT, l, n, g);
    __syncthreads();
  }
  if (a.dal_out != nullptr && (int)blockIdx.x < a.dal_layers && wave == 0) {
    // per-lane strided fp64 sums, then a fixed xor butterfly: the same order on every call
    double sd = 0.0;
    if constexpr (MODE == 1) {
      const float* pp = a.dal_part + (int64_t)blockIdx.x * a.dal_n;
      for (int64_t x = l; x < a.dal_n; x += 64) sd += (double)pp[x];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sd += __shfl_xor(sd, off);
    }
    if (l == 0) a.dal_out[blockIdx.x] = (float)sd;
  }
}

template <int MODE, int NC, int NF, bool DEV>
hipError_t launch(const BkArgs& a, unsigned blocks, hipStream_t s) {
  const size_t smem = sizeof(BkSmem);
  static std::atomic<uint32_t> lds_set{0};
  hipError_t e = ensure_lds_limit(bwdk_ring_kernel<MODE, NC, NF, DEV>, lds_set, (int)smem);
  if (e != hipSuccess) return e;
  bwdk_ring_kernel<MODE, NC, NF, DEV><<<blocks, 512, smem, s>>>(a);
  return hipGetLastError();
}

template <int MODE, int NC, bool DEV>
hipError_t launch_far(const BkArgs& a, int n_far, unsigned blocks, hipStream_t s) {
  switch (n_far) {
    case 0: return launch<MODE, NC, 0, DEV>(a, blocks, s);
    case 1: return launch<MODE, NC, 1, DEV>(a, blocks, s);
    case 2: return launch<MODE, NC, 2, DEV>(a, blocks, s);
    default: return launch<MODE, NC, 3, DEV>(a, blocks, s);
  }
}

constexpr int kMaxFarK = 3;  // far offsets whose rows fit the registers at 8 waves

// covered and far counts (with alpha in device memory: bounds over the alpha range)
void split(const BwdArgs& f, int* n_cov, int* n_far) {
  if (f.plan != nullptr) {
    range_counts(f.alpha_lo, f.alpha_hi, f.base, f.n_base, f.W, f.mode, f.N, 8, n_cov, n_far);
  } else {
    split_table(f.tab, f.N, 8, n_cov, n_far);
  }
}

}  // namespace

bool bwdk_ring_supported(const BwdArgs& f) {
  if (f.dtype != 1 || f.W > kMaxBand || f.N > (1LL << 30)) return false;
  int cov, far;
  split(f, &cov, &far);
  return far <= kMaxFarK && cov <= kMaxCov;
}

int bwdk_instance_key(const BwdArgs& f) {
  if (!bwdk_ring_supported(f)) return -1;
  int cov, far;
  split(f, &cov, &far);
  return (cov <= 8 ? 8 : 16) * 10 + far;
}

hipError_t launch_bwdk_ring(const BwdArgs& f, const float* delta, const uint32_t* ps, const float* dal_part,
                            int64_t dal_n, const bf16_t* qr, const bf16_t* kr) {
  if (f.mode == 1 && ps == nullptr) return hipErrorInvalidValue;
  BkArgs a;
  a.dal_part = dal_part;
  a.dal_n = dal_n;
  a.dal_out = f.dalpha;
  a.dal_layers = f.layers;
  a.q = (const bf16_t*)f.q;
  a.k = (const bf16_t*)f.k;
  a.v = (const bf16_t*)f.v;
  a.dout = (const bf16_t*)f.dout;
  a.lse = f.lse;
  a.delta = delta;
  a.ps = ps;
  a.ps_slots = f.ps_slots;
  a.qr = qr;
  a.kr = kr;
  a.dk = (bf16_t*)f.dk;
  a.dv = (bf16_t*)f.dv;
  a.N = (int)f.N;
  a.W = f.W;
  int n_far;
  split(f, &a.n_cov, &n_far);
  a.plan = f.plan;
  a.n_far = n_far;
  a.heads_per_plan = f.heads_per_plan;
  for (int e = 0; e < kMaxCov; ++e) {
    a.dist[e] = e < a.n_cov ? f.tab.dist[e] : kMaxBand;
    a.w[e] = e < a.n_cov ? f.tab.w[e] : 0.f;
  }
  for (int x = 0; x < kMaxFar; ++x) {
    a.far_dist[x] = x < n_far ? f.tab.dist[a.n_cov + x] : 0;
    a.far_w[x] = x < n_far ? f.tab.w[a.n_cov + x] : 0.f;
  }
  constexpr int kT = step_rows(8);
  // After step p0's insert the ring holds the query rows [p0 + lead - (kP - kT), p0 + lead + kT);
  // the step reads rows p0 .. p0 + kT - 1 + max(covered offset, band): lead is the largest
  // covered offset rounded up to a step (<= kP - kT, the ring reach)
  int need = kMaxBand;
  for (int e = 0; e < a.n_cov; ++e) need = f.tab.dist[e] > need ? f.tab.dist[e] : need;
  a.lead = ((need + kT - 1) / kT) * kT;
  const int64_t tiles = (f.N + kT - 1) / kT;
  const int64_t segs = ring_segments(f.BH, tiles);
  a.seg_len = (int)(((tiles + segs - 1) / segs) * kT);
  a.segs = (int)segs;
  a.scale = (float)(1.0 / sqrt((double)kD));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kD));
  a.rope = f.rope;
  const unsigned blocks = (unsigned)(segs * f.BH);
  if (f.plan != nullptr) {
    if (f.mode == 0)
      return a.n_cov <= 8 ? launch_far<0, 8, true>(a, n_far, blocks, f.stream)
                          : launch_far<0, 16, true>(a, n_far, blocks, f.stream);
    return a.n_cov <= 8 ? launch_far<1, 8, true>(a, n_far, blocks, f.stream)
                        : launch_far<1, 16, true>(a, n_far, blocks, f.stream);
  }
  if (f.mode == 0)
    return a.n_cov <= 8 ? launch_far<0, 8, false>(a, n_far, blocks, f.stream)
                        : launch_far<0, 16, false>(a, n_far, blocks, f.stream);
  return a.n_cov <= 8 ? launch_far<1, 8, false>(a, n_far, blocks, f.stream)
                      : launch_far<1, 16, false>(a, n_far, blocks, f.stream);
}

}  // namespace fib
