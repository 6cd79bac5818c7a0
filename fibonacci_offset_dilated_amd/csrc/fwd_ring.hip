// Fast forward kernel of Fibonacci-offset dilated sparse attention: bf16, D = 64, W <= 16,
// integer and interpolated offsets.
//
// Operation ("Depth-Staggered Fibonacci Spacing for Sparse Attention", gist.science summaries
// of arXiv 2606.28560, Method > Architecture and attention mechanism): query i attends the
// window rows i-W+1..i and one row (integer mode) or one interpolated pair of rows
// (interpolated mode) per table entry, after RoPE. Results 2 notes that static offsets allow
// a fused path; here both modes run fused in this kernel.
//
// Design (gfx950):
//  * One workgroup per CU (8 waves, two per SIMD to cover latencies) sweeps a contiguous
//    segment of one head
//    in steps of 16 queries per wave; wave w owns queries p0 + 16w .. + 15.
//  * LDS ring of the last kP rows: K rotated by RoPE (bf16) and raw V (bf16). Each row is
//    loaded from HBM and rotated once, when it enters the ring; the window band and every
//    table entry whose distance is <= kP - (rows per step) read it from LDS afterwards.
//  * Logits on MFMA as S^T = K^ Q^T (v_mfma_f32_16x16x32_bf16; A = 16 key rows from the ring,
//    B = the wave's 16 rotated queries). The window band is a 32-key by 16-query block; a
//    table entry is a 16-row slab whose diagonal holds the 16 logits (query n reads slab
//    row n), picked out of the lanes that own it.
//  * Table entries beyond the ring read raw K and V rows from global memory, prefetched one
//    step ahead into registers, and use relative RoPE <R_i q, R_(i-d) k> = <R_d q, k> with
//    cos/sin of R_d computed once per workgroup; their P V runs on VALU (v_dot2_f32_bf16).
//  * Long segments: up to two entries (integer mode; one in interpolated mode) a few steps
//    beyond the ring reach are "queued": each step copies the slab (rotated K, V) that the
//    step `depth` steps ahead needs from the ring into registers while its rows are still
//    there, so those rows are read from memory once instead of again per entry. The registers
//    of 8 waves hold two steps of one entry's K and V and five of a second entry's K (its V
//    rows come from global memory); an interpolated entry's slabs are its lower rows plus one
//    dword per lane of the row after them, as a far entry's. A segment's first `depth` steps
//    load their slabs from global memory.
//  * Softmax over all logits of a query at once (they fit in registers), fp32, base 2; the
//    four lanes of a query combine through v_permlane16/32_swap. Logits outside a query's
//    attended set are replaced (selected) by -inf, never offset, so a non-finite K row
//    reaches exactly the queries that attend it.
//  * P V on MFMA as O^T = V^T P^T: V^T operands come from the ring through the LDS transpose
//    read (ds_read_b64_tr_b16); table entries use a diagonal P^T block, two slabs per MFMA
//    (integer mode: two entries; interpolated mode: the lower and upper slab of one entry,
//    weights 1-w and w), built with v_perm_b32 from one packed pair of bf16 weights.
//  * Output dimensions are permuted so that a lane's 16 accumulators are the dims 8g..8g+7
//    and 32+8g..32+8g+7 of its query: V is stored in the ring in that order, far V rows load
//    as two 16-byte pieces and each lane stores two 16-byte pieces of O.
//  * Ring rows are padded to 144 bytes: with 64 LDS banks, 16 consecutive rows then start on 16
//    distinct 4-bank groups, so the A-operand reads (16 rows, one 16-byte chunk each) and the
//    transpose reads (4 rows x 32 bytes per 16 lanes) are conflict-free, and every read of a
//    row is one base address plus immediate offsets.
#include "ring_common.h"

#include <algorithm>

namespace fib {
namespace {

using namespace ring;


struct RingArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  float* lse;
  int N;
  int W;
  int n_cov;        // entries served from the ring (a prefix of the table)
  int early_rows;   // steps whose rows start below this need the position checks
  int seg_len;      // rows per segment (multiple of the step)
  int segs;         // segments per head
  int warm;         // rows inserted before the segment start (multiple of the step)
  float scale_log2;
  int dist[kMaxCov];  // covered distances; slots past n_cov hold a harmless in-ring distance
  float w[kMaxCov];
  int far_dist[kMaxFar];
  float far_w[kMaxFar];
  int unc_dist[kMaxUnc];
  Rope rope;
  const DevPlan* plan;  // alpha in device memory: the split above comes from here (DEV instances)
  int n_far;            // far entries in use (DEV instances: NF is an upper bound)
  int heads_per_plan;   // DEV instances: head h reads plan[h / heads_per_plan]
  int q_dist[kMaxQ];    // queued entries: distances in the queue slots (interpolated: c, one slot)
  float q_w[kMaxQ];     // their weights (interpolated mode)
};

struct __align__(16) Smem {
  uint8_t ringK[(kP + kMirror) * kRow];
  uint8_t ringV[(kP + kMirror) * kRow];
  float2 unc_cs[kMaxUnc][kHalf];
  float2 base_cs[2][kHalf];
  float2 warm_cs[8][kHalf];  // step bases of the warm-up rows
  float2 q_cs[kQDepth0 + kQDepth1][kHalf];  // bases of the queued slabs loaded from global memory
};

// Rows of the far table entries for one step, held in registers and loaded one step ahead:
// lane (n, g) holds, per far entry, K and V row i0w - d + n, dims 8g..8g+7 and 32+8g..32+8g+7
// (K: the A operand of the logit MFMA; V: the lane's slice of O). In interpolated mode that
// is the lower row; the upper row of query n is the lower row of query n + 1 (upper_rows), and
// the one that no lane holds, row i0w - d + 16, is kept spread over the wave (kex, vex: lane l
// holds its dword l % 32).
template <int NF>
struct FarRows {
  uint4 k[NF > 0 ? NF : 1][2];
  uint4 v[NF > 0 ? NF : 1][2];
  uint32_t kex[NF > 0 ? NF : 1];
  uint32_t vex[NF > 0 ? NF : 1];
};

// n_use: far slots in use (NF, or fewer in DEV instances: the unused slots are zero-filled
// without a load; n_use is wave-uniform, so the test is a scalar branch)
template <int MODE, int NF>
__device__ __forceinline__ void load_far_k(const int* fdist, int n_use, FarRows<NF>& fr, const RingArgs& a,
                                           const bf16_t* Kh, int i0w, int l, int n, int g, int lane_off) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f >= n_use) {
      fr.k[f][0] = fr.k[f][1] = make_uint4(0, 0, 0, 0);
      fr.kex[f] = 0u;
      continue;
    }
    const bf16_t* kp = Kh + far_off(fdist[f], i0w, n, g, lane_off);
    fr.k[f][0] = *reinterpret_cast<const uint4*>(kp);
    fr.k[f][1] = *reinterpret_cast<const uint4*>(kp + kHalf);
    if (MODE == 1) {
      // row i0w - d + 16 (< N: far distances exceed the ring reach); rows before 0 only meet
      // masked queries
      const int r = i0w - fdist[f] + 16;
      fr.kex[f] = reinterpret_cast<const uint32_t*>(Kh + (int64_t)(r > 0 ? r : 0) * kD)[l & 31];
    }
  }
}

template <int MODE, int NF>
__device__ __forceinline__ void load_far_v(const int* fdist, int n_use, FarRows<NF>& fr, const RingArgs& a,
                                           const bf16_t* Vh, int i0w, int l, int n, int g, int lane_off) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f >= n_use) {
      fr.v[f][0] = fr.v[f][1] = make_uint4(0, 0, 0, 0);
      fr.vex[f] = 0u;
      continue;
    }
    const bf16_t* vp = Vh + far_off(fdist[f], i0w, n, g, lane_off);
    fr.v[f][0] = *reinterpret_cast<const uint4*>(vp);
    fr.v[f][1] = *reinterpret_cast<const uint4*>(vp + kHalf);
    if (MODE == 1) {
      const int r = i0w - fdist[f] + 16;
      fr.vex[f] = reinterpret_cast<const uint32_t*>(Vh + (int64_t)(r > 0 ? r : 0) * kD)[l & 31];
    }
  }
}

// acc[mb][v] += weights x V, one far row (or row pair) of the lane's 16 output dims: acc[0]
// and acc[1] are dims 8g..8g+3 and 8g+4..8g+7 (x0 = first 16 bytes), acc[2] and acc[3] the
// dims 32 + the same (x1). Integer mode: w0 = (p, 0) and w1 = (0, p) pick one element of a
// bf16 pair. Interpolated mode: the lower and upper row's element of a dim are paired and
// dotted with (p (1-w), p w).
__device__ __forceinline__ void far_pv_int(f4* acc, uint4 x0, uint4 x1, uint32_t w0, uint32_t w1) {
  const uint32_t e[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    acc[mb][0] = dot2(e[2 * mb], w0, acc[mb][0]);
    acc[mb][1] = dot2(e[2 * mb], w1, acc[mb][1]);
    acc[mb][2] = dot2(e[2 * mb + 1], w0, acc[mb][2]);
    acc[mb][3] = dot2(e[2 * mb + 1], w1, acc[mb][3]);
  }
}
__device__ __forceinline__ void far_pv_interp(f4* acc, uint4 x0, uint4 x1, uint4 y0, uint4 y1, uint32_t wp) {
  const uint32_t e[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  const uint32_t h[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    acc[mb][0] = dot2(__builtin_amdgcn_perm(h[2 * mb], e[2 * mb], 0x05040100u), wp, acc[mb][0]);
    acc[mb][1] = dot2(__builtin_amdgcn_perm(h[2 * mb], e[2 * mb], 0x07060302u), wp, acc[mb][1]);
    acc[mb][2] = dot2(__builtin_amdgcn_perm(h[2 * mb + 1], e[2 * mb + 1], 0x05040100u), wp, acc[mb][2]);
    acc[mb][3] = dot2(__builtin_amdgcn_perm(h[2 * mb + 1], e[2 * mb + 1], 0x07060302u), wp, acc[mb][3]);
  }
}

// NQ: queued entries (integer mode 0, 1 or 2; interpolated mode 0 or 1): the table entries
// after the covered ones, within queue_fits of depth kQDepth0 (slot 0) and kQDepth1 (slot 1)
template <int MODE, int NC, int NF, int WAVES, bool DEV, int NQ>
__global__ __launch_bounds__(64 * WAVES, 1) void fwd_ring_kernel(RingArgs a) {
  static_assert(NQ == 0 || (!DEV && (MODE == 0 || NQ == 1)), "queued entries: alpha on the host");
  constexpr int kThreads = 64 * WAVES;
  constexpr int kT = step_rows(WAVES);
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int n = l & 15;   // query (and row) within the wave's 16
  const int g = l >> 4;   // lane group: dims 8g..8g+7 and 32+8g..32+8g+7
  const bool diag_lane = g == (n >> 2);
  const int jr = n >> 2;  // transpose-read row within a 4-row group
  const int jc = n & 3;   // transpose-read 4-column group

  const int N = a.N;
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
  auto S_far_dist = [&](int x) -> int { if constexpr (DEV) return lcl.far_dist[x]; else return a.far_dist[x]; };
  auto S_far_w = [&](int x) -> float { if constexpr (DEV) return lcl.far_w[x]; else return a.far_w[x]; };

  // ---- per-launch set-up: cos/sin of the far distances; per-lane rotation by t = 16 wave + n
  // (the row's offset from a step base)
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
  // masks (selects, not additive biases, so that a NaN logit of a key that a query does not
  // attend stays out of its softmax): window keys by distance (band key kappa of the lane at
  // distance n + 16 - 4g - v in block 0 and n - 4g - v in block 1); table entries are kept in
  // the diagonal lanes only
  bool in0[4], in1[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int d0 = n + 16 - 4 * g - v, d1 = n - 4 * g - v;
    in0[v] = d0 < a.W;
    in1[v] = d1 >= 0 && d1 < a.W;
  }
  // byte selectors of diag_block: slot s = l & 3 of slab A (lo half of x) and slab B (hi half)
  uint32_t sel[4];
  {
    const uint32_t zero = 0x0c0c0c0cu;
    const uint32_t a_half = (l & 1) ? 0x01000c0cu : 0x0c0c0100u;
    const uint32_t b_half = (l & 1) ? 0x03020c0cu : 0x0c0c0302u;
    const bool low = (l & 2) == 0;
    sel[0] = low ? a_half : zero;
    sel[1] = low ? zero : a_half;
    sel[2] = low ? b_half : zero;
    sel[3] = low ? zero : b_half;
  }
  // ds_bpermute address of the query's diagonal lane
  const int diag_addr = 4 * (16 * (n >> 2) + n);
  // lane parts of the LDS addresses: slab reads (row n, chunk g) and transpose reads (row
  // 4g + jr, ring positions 4 jc..)
  const int lane_k = n * kRow + 16 * g;
  const int lane_v = (4 * g + jr) * kRow + 8 * jc;
  // element offset of the lane's part of a 16-row slab: row n, dims 8g.. (and 32+8g..)
  const int lane_off = n * kD + 8 * g;
  // queued V reads: row n, ring positions 4g, 16 + 4g, 32 + 4g, 48 + 4g (dims 8g..8g+7 and
  // 32+8g..32+8g+7 in the order of a far V row)
  const int lane_vq = n * kRow + 8 * g;

  // stores row rb + n of the lane (rb wave-uniform): K^ as given; V in output order, dims
  // 8g..8g+3 | 8g+4.. | 32+8g.. | 36+8g.. at ring positions 4g, 16+4g, 32+4g, 48+4g
  auto put_row = [&](int rb, uint4 kr0, uint4 kr1, uint4 v0, uint4 v1) {
    const int slot = rb & (kP - 1);
    auto put = [&](int ro) {
      uint8_t* kp = sm.ringK + ro + 16 * g;
      uint8_t* vp = sm.ringV + ro + 8 * g;
      lds_write16(kp, 0, kr0);
      lds_write16(kp, 64, kr1);
      lds_write8(vp, 0, v0.x, v0.y);
      lds_write8(vp, 32, v0.z, v0.w);
      lds_write8(vp, 64, v1.x, v1.y);
      lds_write8(vp, 96, v1.z, v1.w);
    };
    put((slot + n) * kRow);
    if (slot < kMirror) put((slot + kP + n) * kRow);  // mirrored rows are stored twice
  };

  const int64_t head = blockIdx.x / a.segs;
  const int seg = blockIdx.x % a.segs;
  const int s0 = seg * a.seg_len;
  const int s1 = s0 + a.seg_len < N ? s0 + a.seg_len : N;
  const size_t hoff = (size_t)head * (size_t)N * kD;
  const bf16_t* Qh = a.q + hoff;
  const bf16_t* Kh = a.k + hoff;
  const bf16_t* Vh = a.v + hoff;

  // rows this lane inserts: q/k/v dims 8g.. and 32+8g.. of row pb + 16w + n. Rows past the
  // end repeat row N - 1: only queries past the end read them.
  auto load_rows = [&](int pb, uint4* q2, uint4* k2, uint4* v2) {
    const int rb = pb + 16 * wave;
    int64_t off;
    if (rb + 15 < N) {
      off = (int64_t)rb * kD + lane_off;
    } else {
      const int r = rb + n < N ? rb + n : N - 1;
      off = (int64_t)r * kD + 8 * g;
    }
    const bf16_t* qp = Qh + off;
    const bf16_t* kp = Kh + off;
    const bf16_t* vp = Vh + off;
    q2[0] = *reinterpret_cast<const uint4*>(qp);
    q2[1] = *reinterpret_cast<const uint4*>(qp + kHalf);
    k2[0] = *reinterpret_cast<const uint4*>(kp);
    k2[1] = *reinterpret_cast<const uint4*>(kp + kHalf);
    v2[0] = *reinterpret_cast<const uint4*>(vp);
    v2[1] = *reinterpret_cast<const uint4*>(vp + kHalf);
  };

  // ---- warm-up: ring rows [ws, s0), the band and covered rows of the first steps. Rows
  // before 0 are never stored: their slots must read as zero (finite, and masked).
  const int ws = s0 - S_warm > 0 ? s0 - S_warm : 0;
  const int n_warm = (s0 - ws) / kT;  // whole steps (s0 and the warm-up are step multiples)
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
  if constexpr (NQ > 0) {
    // slab x of slot 0 (x < kQDepth0), then of slot 1: rows s0 + x T - d + 16w + n
    constexpr int n_qs = NQ > 1 ? kQDepth0 + kQDepth1 : kQDepth0;
    for (int x = tid; x < n_qs * kHalf; x += kThreads) {
      const int u = x / kHalf, t = x % kHalf;
      const int base = u < kQDepth0 ? s0 + kT * u - a.q_dist[0] : s0 + kT * (u - kQDepth0) - a.q_dist[1];
      sm.q_cs[u][t] = rope_cs(base, a.rope.rev[t]);
    }
  }
  uint4 pq[2], pk[2], pv[2];
  load_rows(s0, pq, pk, pv);
  __syncthreads();
  {
    // kWB steps of warm rows in flight at once: K rotated by R_(base + t), V as loaded
    constexpr int kWB = WAVES == 8 ? 3 : 4;
    for (int j0 = 0; j0 < n_warm; j0 += kWB) {
      uint4 wk[kWB][2], wv[kWB][2];
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          const int64_t off = (int64_t)(ws + (j0 + jj) * kT + 16 * wave) * kD + lane_off;
          wk[jj][0] = *reinterpret_cast<const uint4*>(Kh + off);
          wk[jj][1] = *reinterpret_cast<const uint4*>(Kh + off + kHalf);
          wv[jj][0] = *reinterpret_cast<const uint4*>(Vh + off);
          wv[jj][1] = *reinterpret_cast<const uint4*>(Vh + off + kHalf);
        }
      }
#pragma unroll
      for (int jj = 0; jj < kWB; ++jj) {
        if (j0 + jj < n_warm) {
          float2 cs[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float2 b = sm.warm_cs[j0 + jj][8 * g + t];
            cs[t] = make_float2(b.x * cs_t[t].x - b.y * cs_t[t].y, b.y * cs_t[t].x + b.x * cs_t[t].y);
          }
          float kf[16];
          unpack8(wk[jj][0], kf);
          unpack8(wk[jj][1], kf + 8);
          uint4 kr0, kr1;
          rotate_pack_f(kf, cs, &kr0, &kr1);
          put_row(ws + (j0 + jj) * kT + 16 * wave, kr0, kr1, wv[jj][0], wv[jj][1]);
        }
      }
    }
  }
  // (the first step's barrier orders these stores before any read of them)
  // far K rows of the first step (requested after the warm-up rows, whose registers they reuse)
  FarRows<NF> fr;
  load_far_k<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fr, a, Kh, s0 + 16 * wave, l, n, g,
                       lane_off);
  if constexpr (MODE == 0)
    load_far_v<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fr, a, Vh, s0 + 16 * wave, l, n, g,
                         lane_off);

  // ---- queued entries: slab x of a slot serves the step x steps ahead (x = 0: this step).
  // Those of the segment's first steps come from global memory (raw rows, K rotated here by
  // its row's position); each later one is read from the ring, `depth` steps before its use.
  // Lane (n, g) holds row n: K^ as a logit A operand, V as a far V row (dims 8g.. and 32+8g..).
  // Slot 1 queues only K (the registers of 8 waves hold no more); its V rows are loaded from
  // global memory one step ahead, as a far entry's.
  uint4 qk0[kQDepth0][2], qv0[kQDepth0][2], qk1[kQDepth1][2], qv1[2];
  // interpolated mode (slot 0): the slabs are the lower rows c back; the upper rows come from
  // the neighbouring lane and the row after the slab, held one dword per lane (as a far
  // entry's): dword l % 32 of K^ and of V (in the natural dim order)
  uint32_t qkx0[kQDepth0], qvx0[kQDepth0];
  // byte offset of V dword l % 32 (dims 2j, 2j + 1) in a ring row (output order)
  const int vex_off = [&] {
    const int j = l & 31, jj = j & 15, t = jj & 3;
    return 64 * (j >> 4) + 8 * (jj >> 2) + (t < 2 ? 4 * t : 32 + 4 * (t - 2));
  }();
  // rows pb + 16w - d + n (pb: a step's first row)
  auto q_global = [&](int d, int pb, uint4* k2, uint4* v2) {
    const int64_t off = far_off(d, pb + 16 * wave, n, g, lane_off);
    k2[0] = *reinterpret_cast<const uint4*>(Kh + off);
    k2[1] = *reinterpret_cast<const uint4*>(Kh + off + kHalf);
    if (v2 != nullptr) {
      v2[0] = *reinterpret_cast<const uint4*>(Vh + off);
      v2[1] = *reinterpret_cast<const uint4*>(Vh + off + kHalf);
    }
  };
  auto q_global_v = [&](int d, int pb, uint4* v2) {
    const int64_t off = far_off(d, pb + 16 * wave, n, g, lane_off);
    v2[0] = *reinterpret_cast<const uint4*>(Vh + off);
    v2[1] = *reinterpret_cast<const uint4*>(Vh + off + kHalf);
  };
  // rotation by R_(base + 16w + n), base cos/sin from q_cs[u] (rows before 0 only meet masked
  // queries; far_off loaded row 0 for them)
  auto q_rotate = [&](int u, uint4* k2) {
    float2 cs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 b = sm.q_cs[u][8 * g + t];
      cs[t] = make_float2(b.x * cs_t[t].x - b.y * cs_t[t].y, b.y * cs_t[t].x + b.x * cs_t[t].y);
    }
    float kf[16];
    unpack8(k2[0], kf);
    unpack8(k2[1], kf + 8);
    rotate_pack_f(kf, cs, &k2[0], &k2[1]);
  };
  // interpolated: the row after the slab (pb + 16w - c + 16), dword l % 32 of K (rotated by
  // its position with its RoPE partner dword l % 32 ^ 16) and of V
  auto q_global_ex = [&](int c, int pb, uint32_t* kx, uint32_t* vx) {
    const int r = pb + 16 * wave - c + 16;
    const int64_t ro = (int64_t)(r > 0 ? r : 0) * kD;  // (rows before 0 only meet masked queries)
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(Kh + ro);
    const int j = l & 31;
    const uint32_t x = kr[j], y = kr[j ^ 16];
    *vx = reinterpret_cast<const uint32_t*>(Vh + ro)[j];
    const int m = 2 * (j & 15);
    const float2 c0 = rope_cs(r, a.rope.rev[m]), c1 = rope_cs(r, a.rope.rev[m + 1]);
    const float sg = j < 16 ? -1.f : 1.f;  // x'_m = x_m c - x_(m+32) s; x'_(m+32) = x_(m+32) c + x_m s
    *kx = pack_bf2(bf_lo(x) * c0.x + sg * bf_lo(y) * c0.y, bf_hi(x) * c1.x + sg * bf_hi(y) * c1.y);
  };
  // rows rb - d + n (rb: this wave's first row of a step) from the ring
  auto q_ring = [&](int d, int rb, uint4* k2, uint4* v2) {
    const int ro = row_off(rb - d);
    k2[0] = lds_read16(sm.ringK, ro + lane_k);
    k2[1] = lds_read16(sm.ringK, ro + lane_k + 64);
    if (v2 == nullptr) return;
    const int vo = ro + lane_vq;
    const uint2 x0 = lds_read8(sm.ringV, vo), x1 = lds_read8(sm.ringV, vo + 32);
    const uint2 x2 = lds_read8(sm.ringV, vo + 64), x3 = lds_read8(sm.ringV, vo + 96);
    v2[0] = make_uint4(x0.x, x0.y, x1.x, x1.y);
    v2[1] = make_uint4(x2.x, x2.y, x3.x, x3.y);
  };
  auto q_ring_ex = [&](int c, int rb, uint32_t* kx, uint32_t* vx) {
    const int ro = row_off(rb - c + 16);
    *kx = lds_read4(sm.ringK, ro + 4 * (l & 31));
    *vx = lds_read4(sm.ringV, ro + vex_off);
  };
  if constexpr (NQ > 0) {
#pragma unroll
    for (int x = 0; x < kQDepth0; ++x) q_global(a.q_dist[0], s0 + kT * x, qk0[x], qv0[x]);
    if constexpr (MODE == 1) {
#pragma unroll
      for (int x = 0; x < kQDepth0; ++x) q_global_ex(a.q_dist[0], s0 + kT * x, &qkx0[x], &qvx0[x]);
    }
    if constexpr (NQ > 1) {
#pragma unroll
      for (int x = 0; x < kQDepth1; ++x) q_global(a.q_dist[1], s0 + kT * x, qk1[x], nullptr);
      q_global_v(a.q_dist[1], s0, qv1);
    }
#pragma unroll
    for (int x = 0; x < kQDepth0; ++x) q_rotate(x, qk0[x]);
    if constexpr (NQ > 1) {
#pragma unroll
      for (int x = 0; x < kQDepth1; ++x) q_rotate(kQDepth0 + x, qk1[x]);
    }
    // Interpolated mode: the raw rows loaded here are made ready before the step loop (an
    // empty asm that reads them). Left in flight into the loop, the moves of its queue at each
    // step's start would wait for every load in flight. (The integer instances have no such
    // moves, and there the asm costs them their register fit.)
    if constexpr (MODE == 1) {
      auto ready = [](uint4& v) { asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); };
#pragma unroll
      for (int x = 0; x < kQDepth0; ++x) {
        ready(qv0[x][0]);
        ready(qv0[x][1]);
        asm volatile("" : "+v"(qkx0[x]), "+v"(qvx0[x]));
      }
    }
  }

  int buf = 0;
  for (int p0 = s0; p0 < s1; p0 += kT, buf ^= 1) {
    // ---- insert rows p0 + 16w + n: rotate K (and Q for this step's queries) by R_(p0 + t)
    float2 cs[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float2 b = sm.base_cs[buf][8 * g + t];
      cs[t] = make_float2(b.x * cs_t[t].x - b.y * cs_t[t].y, b.y * cs_t[t].x + b.x * cs_t[t].y);
    }
    float qf[16], kf[16];
    unpack8(pq[0], qf);
    unpack8(pq[1], qf + 8);
    unpack8(pk[0], kf);
    unpack8(pk[1], kf + 8);
    uint4 kr0, kr1, qh0, qh1;
    rotate_pack_f(kf, cs, &kr0, &kr1);
    rotate_pack_f(qf, cs, &qh0, &qh1);
    const int bw = p0 + 16 * wave;  // row i0w of this wave's queries
    put_row(bw, kr0, kr1, pv[0], pv[1]);
    __syncthreads();
    // next step's rows (the last step loads harmless repeats) and base rotation
    const int pn = p0 + kT;
    load_rows(pn < s1 ? pn : p0, pq, pk, pv);
    if (wave == 0 && l < kHalf) sm.base_cs[buf ^ 1][l] = rope_cs(pn, rev_l);

    {
      const int i0w = p0 + 16 * wave;
      const int iq = i0w + n;  // this lane's query
      const bf16x8 bq0 = as_bf8(qh0), bq1 = as_bf8(qh1);
      // keys before position 0 (and table distances longer than the query position) occur
      // only in the first steps of a sequence; afterwards the masks are the fixed ones above
      const bool early = i0w < S_early_rows;

      // ---- window band: keys i0w - 16 + kappa, kappa < 32
      f4 S0 = {0, 0, 0, 0}, S1 = {0, 0, 0, 0};
      const int band = row_off(bw - 16);  // slab 0 at +0, slab 1 at +16 rows
      {
        const int sa = band + lane_k;
        S0 = mfma32(as_bf8(lds_read16(sm.ringK, sa)), bq0, S0);
        S0 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 64)), bq1, S0);
        S1 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 16 * kRow)), bq0, S1);
        S1 = mfma32(as_bf8(lds_read16(sm.ringK, sa + 16 * kRow + 64)), bq1, S1);
      }
      // ---- covered entries: 16-row slabs from the ring (entries past n_cov are masked)
      float s_ent[NC];
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        const int sl = row_off(bw - S_dist(e)) + lane_k;
        f4 S = {0, 0, 0, 0};
        S = mfma32(as_bf8(lds_read16(sm.ringK, sl)), bq0, S);
        S = mfma32(as_bf8(lds_read16(sm.ringK, sl + 64)), bq1, S);
        float s = sel4(S, l);
        if (MODE == 1) {
          // the upper slab is the next row
          f4 H = {0, 0, 0, 0};
          H = mfma32(as_bf8(lds_read16(sm.ringK, sl + kRow)), bq0, H);
          H = mfma32(as_bf8(lds_read16(sm.ringK, sl + kRow + 64)), bq1, H);
          s = fmaf(S_w(e), sel4(H, l) - s, s);
        }
        s_ent[e] = diag_lane ? s * sl2 : -INFINITY;
      }
      if (S_n_cov < NC) {
#pragma unroll
        for (int e = 0; e < NC; ++e)
          if (e >= S_n_cov) s_ent[e] = -INFINITY;
      }

      // ---- far entries: their K rows were requested at the end of the previous step
      float s_far[NF > 0 ? NF : 1];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int u = MODE == 1 ? 2 * f : f;
        uint4 r0, r1;
        rotate_pack_f(qf, &sm.unc_cs[u][8 * g], &r0, &r1);
        f4 S = {0, 0, 0, 0};
        S = mfma32(as_bf8(fr.k[f][0]), as_bf8(r0), S);
        S = mfma32(as_bf8(fr.k[f][1]), as_bf8(r1), S);
        float s = sel4(S, l);
        if (MODE == 1) {
          rotate_pack_f(qf, &sm.unc_cs[u + 1][8 * g], &r0, &r1);
          f4 H = {0, 0, 0, 0};
          uint4 kh[2];
          upper_rows(fr.k[f], fr.kex[f], g, kh);
          H = mfma32(as_bf8(kh[0]), as_bf8(r0), H);
          H = mfma32(as_bf8(kh[1]), as_bf8(r1), H);
          s = fmaf(S_far_w(f), sel4(H, l) - s, s);
        }
        s_far[f] = diag_lane ? s * sl2 : -INFINITY;
        if (DEV && f >= S_n_far) s_far[f] = -INFINITY;  // slot beyond the table
      }
      // queued entries: slab 0 of each slot
      float s_q[kMaxQ];
      if constexpr (NQ > 0) {
        auto q_logit = [&](const uint4* k2) {
          f4 S = {0, 0, 0, 0};
          S = mfma32(as_bf8(k2[0]), bq0, S);
          S = mfma32(as_bf8(k2[1]), bq1, S);
          return diag_lane ? sel4(S, l) * sl2 : -INFINITY;
        };
        if constexpr (MODE == 0) {
          s_q[0] = q_logit(qk0[0]);
          if constexpr (NQ > 1) s_q[1] = q_logit(qk1[0]);
        } else {
          f4 S = {0, 0, 0, 0}, H = {0, 0, 0, 0};
          S = mfma32(as_bf8(qk0[0][0]), bq0, S);
          S = mfma32(as_bf8(qk0[0][1]), bq1, S);
          uint4 kh[2];
          upper_rows(qk0[0], qkx0[0], g, kh);
          H = mfma32(as_bf8(kh[0]), bq0, H);
          H = mfma32(as_bf8(kh[1]), bq1, H);
          const float lo = sel4(S, l);
          const float sv = fmaf(a.q_w[0], sel4(H, l) - lo, lo);
          s_q[0] = diag_lane ? sv * sl2 : -INFINITY;
        }
      }
      // interpolated: their V rows, for the end of this step (row pairs of K and V are never
      // held together: the registers do not allow it); integer: requested with the K rows
      if constexpr (MODE == 1)
        load_far_v<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fr, a, Vh, i0w, l, n, g, lane_off);


      // ---- softmax over the window band and the entries (base-2 logits)
      float sw0[4], sw1[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sw0[v] = in0[v] ? S0[v] * sl2 : -INFINITY;
        sw1[v] = in1[v] ? S1[v] * sl2 : -INFINITY;
      }
      if (early) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n + 16 - 4 * g - v > iq) sw0[v] = -INFINITY;
#pragma unroll
        for (int e = 0; e < NC; ++e)
          if (S_dist(e) > iq) s_ent[e] = -INFINITY;
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (S_far_dist(f) > iq) s_far[f] = -INFINITY;
#pragma unroll
        for (int x = 0; x < NQ; ++x)
          if (a.q_dist[x] > iq) s_q[x] = -INFINITY;
      }
      float m = fmaxf(fmaxf(sw0[0], sw0[1]), fmaxf(sw0[2], sw0[3]));
#pragma unroll
      for (int v = 0; v < 4; ++v) m = fmaxf(m, sw1[v]);
#pragma unroll
      for (int e = 0; e < NC; ++e) m = fmaxf(m, s_ent[e]);
#pragma unroll
      for (int f = 0; f < NF; ++f) m = fmaxf(m, s_far[f]);
#pragma unroll
      for (int x = 0; x < NQ; ++x) m = fmaxf(m, s_q[x]);
      m = quad_max(m);  // every query has its own key (distance 0), so m is finite
      // lsum: the fp32 sum of the weights, for LSE (each query's weights are spread over its
      // four lanes: window keys in all four, table entries in its diagonal lane)
      float lsum = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        sw0[v] = ex2(sw0[v] - m);
        sw1[v] = ex2(sw1[v] - m);
        lsum += sw0[v] + sw1[v];
      }
#pragma unroll
      for (int e = 0; e < NC; ++e) {
        s_ent[e] = ex2(s_ent[e] - m);
        lsum += s_ent[e];
      }
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        s_far[f] = ex2(s_far[f] - m);
        lsum += s_far[f];
      }
#pragma unroll
      for (int x = 0; x < NQ; ++x) {
        s_q[x] = ex2(s_q[x] - m);
        lsum += s_q[x];
      }
      lsum = quad_add(lsum);

      // ---- P V: O^T[dim][query n], weights in bf16. The normaliser is the sum of exactly the
      // bf16 weights applied (rows of P sum to 1): an all-ones A block adds a fifth output
      // block whose every entry is the column sum of P^T; far weights add through dot2.
      f4 acc[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mb] = f4{0, 0, 0, 0};
      f4 accn = {0, 0, 0, 0};
      const bf16x8 ones = as_bf8(make_uint4(kOnes, kOnes, kOnes, kOnes));
      float lnorm_far = 0.f;
      // transpose reads: lane (jr, jc) of a 16-lane group reads row k0 + jr, ring positions
      // 16 mb + 4 jc .. +3, i.e. bytes 32 mb + 8 jc of the row (k0 = 4g of the slab)
      {
        const bf16x8 bp = __builtin_bit_cast(
            bf16x8, make_uint4(pack_bf2(sw0[0], sw0[1]), pack_bf2(sw0[2], sw0[3]), pack_bf2(sw1[0], sw1[1]),
                               pack_bf2(sw1[2], sw1[3])));
        const int r0 = band + lane_v, r1 = r0 + 16 * kRow;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[mb] = mfma32(cat_bf8(tr16(sm.ringV, r0 + 32 * mb), tr16(sm.ringV, r1 + 32 * mb)), bp, acc[mb]);
        accn = mfma32(ones, bp, accn);
      }
      // covered entries on MFMA with a diagonal P^T block (integer mode: two entries per
      // MFMA, a missing second entry has weight 0 and an in-ring dummy distance; interpolated
      // mode: the lower and upper slab of one entry)
      if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < NC; e += 2) {
          const bf16x8 bp = diag_block(pack_bf2(s_ent[e], s_ent[e + 1]), sel);
          const int ra = row_off(bw - S_dist(e)) + lane_v, rb = row_off(bw - S_dist(e + 1)) + lane_v;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[mb] = mfma32(cat_bf8(tr16(sm.ringV, ra + 32 * mb), tr16(sm.ringV, rb + 32 * mb)), bp, acc[mb]);
          accn = mfma32(ones, bp, accn);
        }
      } else {
#pragma unroll
        for (int e = 0; e < NC; ++e) {
          const float p = s_ent[e];
          const bf16x8 bp = diag_block(pack_bf2(p * (1.f - S_w(e)), p * S_w(e)), sel);
          const int ra = row_off(bw - S_dist(e)) + lane_v, rb = ra + kRow;
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[mb] = mfma32(cat_bf8(tr16(sm.ringV, ra + 32 * mb), tr16(sm.ringV, rb + 32 * mb)), bp, acc[mb]);
          accn = mfma32(ones, bp, accn);
        }
      }

      // far entries on VALU; the weights live in the query's diagonal lane and reach
      // its other three lanes by ds_bpermute, packed two per dword
      if (MODE == 0) {
#pragma unroll
        for (int f = 0; f < NF; f += 2) {
          const uint32_t x = pack_bf2(s_far[f], f + 1 < NF ? s_far[f + 1] : 0.f);
          const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)x);
          lnorm_far = dot2(y, kOnes, lnorm_far);
          far_pv_int(acc, fr.v[f][0], fr.v[f][1], y & 0xffffu, y << 16);
          if (f + 1 < NF) far_pv_int(acc, fr.v[f + 1][0], fr.v[f + 1][1], y >> 16, y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float p = s_far[f];
          const uint32_t x = pack_bf2(p * (1.f - S_far_w(f)), p * S_far_w(f));
          const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)x);
          lnorm_far = dot2(y, kOnes, lnorm_far);
          uint4 vh[2];
          upper_rows(fr.v[f], fr.vex[f], g, vh);
          far_pv_interp(acc, fr.v[f][0], fr.v[f][1], vh[0], vh[1], y);
        }
      }

      // queued entries on VALU as the far ones; then each slot's slabs move one step down and
      // its last one is read from the ring (rows of the step `depth` steps ahead)
      if constexpr (NQ > 0) {
        if constexpr (MODE == 0) {
          const uint32_t x = pack_bf2(s_q[0], NQ > 1 ? s_q[1] : 0.f);
          const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)x);
          lnorm_far = dot2(y, kOnes, lnorm_far);
          far_pv_int(acc, qv0[0][0], qv0[0][1], y & 0xffffu, y << 16);
          if constexpr (NQ > 1) far_pv_int(acc, qv1[0], qv1[1], y >> 16, y & 0xffff0000u);
        } else {
          const float p = s_q[0];
          const uint32_t x = pack_bf2(p * (1.f - a.q_w[0]), p * a.q_w[0]);
          const uint32_t y = (uint32_t)__builtin_amdgcn_ds_bpermute(diag_addr, (int)x);
          lnorm_far = dot2(y, kOnes, lnorm_far);
          uint4 vh[2];
          upper_rows(qv0[0], qvx0[0], g, vh);
          far_pv_interp(acc, qv0[0][0], qv0[0][1], vh[0], vh[1], y);
        }
#pragma unroll
        for (int x2 = 0; x2 + 1 < kQDepth0; ++x2)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            qk0[x2][h] = qk0[x2 + 1][h];
            qv0[x2][h] = qv0[x2 + 1][h];
          }
        q_ring(a.q_dist[0], bw + kT * kQDepth0, qk0[kQDepth0 - 1], qv0[kQDepth0 - 1]);
        if constexpr (MODE == 1) {
#pragma unroll
          for (int x2 = 0; x2 + 1 < kQDepth0; ++x2) {
            qkx0[x2] = qkx0[x2 + 1];
            qvx0[x2] = qvx0[x2 + 1];
          }
          q_ring_ex(a.q_dist[0], bw + kT * kQDepth0, &qkx0[kQDepth0 - 1], &qvx0[kQDepth0 - 1]);
        }
        if constexpr (NQ > 1) {
#pragma unroll
          for (int x2 = 0; x2 + 1 < kQDepth1; ++x2)
#pragma unroll
            for (int h = 0; h < 2; ++h) qk1[x2][h] = qk1[x2 + 1][h];
          q_ring(a.q_dist[1], bw + kT * kQDepth1, qk1[kQDepth1 - 1], nullptr);
        }
      }

      // ---- epilogue: the lane's dims 8g..8g+7 (acc[0], acc[1]) and 32+8g.. (acc[2], acc[3])
      if (iq < s1) {
        const float lnorm = accn[0] + lnorm_far;
        const float inv = 1.f / lnorm;
        bf16_t* op = a.o + hoff + (int64_t)i0w * kD + lane_off;
        uint4 x0, x1;
        x0.x = pack_bf2(acc[0][0] * inv, acc[0][1] * inv);
        x0.y = pack_bf2(acc[0][2] * inv, acc[0][3] * inv);
        x0.z = pack_bf2(acc[1][0] * inv, acc[1][1] * inv);
        x0.w = pack_bf2(acc[1][2] * inv, acc[1][3] * inv);
        x1.x = pack_bf2(acc[2][0] * inv, acc[2][1] * inv);
        x1.y = pack_bf2(acc[2][2] * inv, acc[2][3] * inv);
        x1.z = pack_bf2(acc[3][0] * inv, acc[3][1] * inv);
        x1.w = pack_bf2(acc[3][2] * inv, acc[3][3] * inv);
        *reinterpret_cast<uint4*>(op) = x0;
        *reinterpret_cast<uint4*>(op + kHalf) = x1;
        if (g == 0 && a.lse != nullptr) (a.lse + (size_t)head * N + i0w)[n] = (m + log2f(lsum)) * 0.69314718055994530942f;
      }
      // far K rows of the next step, and in integer mode its far V rows (the last step loads
      // rows that are never used)
      load_far_k<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fr, a, Kh, i0w + kT, l, n, g,
                           lane_off);
      if constexpr (MODE == 0)
        load_far_v<MODE, NF>(DEV ? lcl.far_dist : a.far_dist, DEV ? S_n_far : NF, fr, a, Vh, i0w + kT, l, n, g,
                             lane_off);
      // (with them: requested before the stores, their registers would be copied at the step's
      // end, which waits for the loads)
      if constexpr (NQ > 1) q_global_v(a.q_dist[1], p0 + kT, qv1);
    }
    __syncthreads();
  }
}

// Steps per segment of a launch of BH heads of N rows (ring_segments).
int64_t segment_steps(int64_t BH, int64_t N, int waves) {
  const int kT = step_rows(waves);
  const int64_t tiles = (N + kT - 1) / kT;
  const int64_t segs = ring_segments(BH, tiles);
  return (tiles + segs - 1) / segs;
}

// Waves per workgroup and the table split: 8 waves (two per SIMD). Every instance fits 256
// registers per lane at 8 waves (the interpolated far entries hold only their lower rows).
// With alpha in device memory the counts are upper bounds over the alpha range. Queued
// entries (alpha on the host): the first entries past the covered ones that fit the queue
// slots, when segments are long enough (8 steps) for the ring to serve most of their slabs,
// in the instances that fit the registers. Integer mode: one queued entry with up to two far
// ones, two with up to two (up to 8 covered entries) or one (up to 16); interpolated mode:
// one queued entry with up to two far ones.
int plan(const FwdArgs& f, int* n_cov, int* n_q, int* n_far) {
  *n_q = 0;
  if (f.plan != nullptr) {
    range_counts(f.alpha_lo, f.alpha_hi, f.base, f.n_base, f.W, f.mode, f.N, 8, n_cov, n_far);
    return 8;
  }
  split_table(f.tab, f.N, 8, n_cov, n_far);
  if (f.mode == 1 && segment_steps(f.BH, f.N, 8) >= 8 && *n_cov <= kMaxCov) {
    // interpolated: slot 0 only (with its lower slab, the neighbouring row and up to two far
    // entries the registers are full)
    if (*n_far >= 1 && *n_far <= 3 && queue_fits_interp(f.tab.dist[*n_cov], kQDepth0, 8)) {
      *n_q = 1;
      *n_far -= 1;
    }
    return 8;
  }
  if (f.mode == 0 && segment_steps(f.BH, f.N, 8) >= 8 && *n_cov <= kMaxCov) {
    const int c = *n_cov;
    int q = 0;
    if (*n_far >= 1 && queue_fits(f.tab.dist[c], kQDepth0, 8)) {
      q = 1;
      if (*n_far >= 2 && queue_fits(f.tab.dist[c + 1], kQDepth1, 8)) q = 2;
    }
    for (; q > 0; --q) {
      const int rest = *n_far - q;
      if (rest <= (q == 2 && c > 8 ? 1 : 2)) break;
    }
    *n_q = q;
    *n_far -= q;
  }
  return 8;
}

template <int MODE, int NC, int NF, int WAVES, bool DEV, int NQ>
hipError_t launch(const RingArgs& a, unsigned blocks, hipStream_t s) {
  const size_t smem = sizeof(Smem);
  static std::atomic<uint32_t> lds_set{0};
  hipError_t e = ensure_lds_limit(fwd_ring_kernel<MODE, NC, NF, WAVES, DEV, NQ>, lds_set, (int)smem);
  if (e != hipSuccess) return e;
  fwd_ring_kernel<MODE, NC, NF, WAVES, DEV, NQ><<<blocks, 64 * WAVES, smem, s>>>(a);
  return hipGetLastError();
}

// kernel instance by (covered entries rounded up to 8 or 16, far entries, waves); with alpha
// in device memory (DEV) the counts are bounds over the alpha range
template <int MODE, int WAVES, bool DEV = false>
hipError_t launch_mode(const RingArgs& a, int n_far, unsigned blocks, hipStream_t s) {
  if (a.n_cov <= 8) {
    switch (n_far) {
      case 0: return launch<MODE, 8, 0, WAVES, DEV, 0>(a, blocks, s);
      case 1: return launch<MODE, 8, 1, WAVES, DEV, 0>(a, blocks, s);
      case 2: return launch<MODE, 8, 2, WAVES, DEV, 0>(a, blocks, s);
      case 3: return launch<MODE, 8, 3, WAVES, DEV, 0>(a, blocks, s);
      default: return launch<MODE, 8, 4, WAVES, DEV, 0>(a, blocks, s);
    }
  }
  switch (n_far) {
    case 0: return launch<MODE, 16, 0, WAVES, DEV, 0>(a, blocks, s);
    case 1: return launch<MODE, 16, 1, WAVES, DEV, 0>(a, blocks, s);
    case 2: return launch<MODE, 16, 2, WAVES, DEV, 0>(a, blocks, s);
    case 3: return launch<MODE, 16, 3, WAVES, DEV, 0>(a, blocks, s);
    default: return launch<MODE, 16, 4, WAVES, DEV, 0>(a, blocks, s);
  }
}

// integer mode with queued entries (the combinations plan() picks)
template <int NC>
hipError_t launch_queued_nc(const RingArgs& a, int n_q, int n_far, unsigned blocks, hipStream_t s) {
  if (n_q == 1) {
    switch (n_far) {
      case 0: return launch<0, NC, 0, 8, false, 1>(a, blocks, s);
      case 1: return launch<0, NC, 1, 8, false, 1>(a, blocks, s);
      default: return launch<0, NC, 2, 8, false, 1>(a, blocks, s);
    }
  }
  switch (n_far) {
    case 0: return launch<0, NC, 0, 8, false, 2>(a, blocks, s);
    case 1: return launch<0, NC, 1, 8, false, 2>(a, blocks, s);
    default:
      if constexpr (NC == 8) return launch<0, NC, 2, 8, false, 2>(a, blocks, s);
      return hipErrorInvalidValue;  // (not picked)
  }
}
template <int NC>
hipError_t launch_queued_interp_nc(const RingArgs& a, int n_far, unsigned blocks, hipStream_t s) {
  switch (n_far) {
    case 0: return launch<1, NC, 0, 8, false, 1>(a, blocks, s);
    case 1: return launch<1, NC, 1, 8, false, 1>(a, blocks, s);
    default: return launch<1, NC, 2, 8, false, 1>(a, blocks, s);
  }
}
hipError_t launch_queued(const RingArgs& a, int mode, int n_q, int n_far, unsigned blocks, hipStream_t s) {
  if (mode == 1)
    return a.n_cov <= 8 ? launch_queued_interp_nc<8>(a, n_far, blocks, s)
                        : launch_queued_interp_nc<16>(a, n_far, blocks, s);
  return a.n_cov <= 8 ? launch_queued_nc<8>(a, n_q, n_far, blocks, s)
                      : launch_queued_nc<16>(a, n_q, n_far, blocks, s);
}

}  // namespace

bool fwd_ring_supported(const FwdArgs& f) {
  if (f.dtype != 1 || f.W > kMaxBand || f.N > (1LL << 30)) return false;
  int cov, q, far;
  plan(f, &cov, &q, &far);
  return q + far <= kMaxFar && cov <= kMaxCov;
}

// (layer stacks group consecutive layers by this key and launch each group with the split
// from the alpha range, which queues no entries: queued and far entries count alike here)
int fwd_instance_key(const FwdArgs& f) {
  if (!fwd_ring_supported(f)) return -1;
  int cov, q, far;
  const int waves = plan(f, &cov, &q, &far);
  return waves * 1000 + (cov <= 8 ? 8 : 16) * 10 + q + far;
}

hipError_t launch_fwd_ring(const FwdArgs& f) {
  RingArgs a;
  a.plan = f.plan;
  a.q = (const bf16_t*)f.q;
  a.k = (const bf16_t*)f.k;
  a.v = (const bf16_t*)f.v;
  a.o = (bf16_t*)f.o;
  a.lse = f.lse;
  a.N = (int)f.N;
  a.W = f.W;
  int n_q, n_far;
  const int waves = plan(f, &a.n_cov, &n_q, &n_far);  // 8
  for (int e = 0; e < kMaxCov; ++e) {
    // slots past the covered prefix get a harmless in-ring distance and weight 0
    a.dist[e] = e < a.n_cov ? f.tab.dist[e] : kMaxBand;
    a.w[e] = e < a.n_cov ? f.tab.w[e] : 0.f;
  }
  // queued entries follow the covered ones in the table, far entries follow those
  for (int x = 0; x < kMaxQ; ++x) {
    a.q_dist[x] = x < n_q ? f.tab.dist[a.n_cov + x] : 0;
    a.q_w[x] = x < n_q ? f.tab.w[a.n_cov + x] : 0.f;
  }
  const int c = a.n_cov + n_q;
  for (int x = 0; x < kMaxFar; ++x) {
    a.far_dist[x] = x < n_far ? f.tab.dist[c + x] : 0;
    a.far_w[x] = x < n_far ? f.tab.w[c + x] : 0.f;
  }
  int u = 0;
  for (int x = 0; x < n_far; ++x) {
    a.unc_dist[u++] = a.far_dist[x];
    if (f.mode == 1) a.unc_dist[u++] = a.far_dist[x] - 1;
  }
  for (; u < kMaxUnc; ++u) a.unc_dist[u] = 0;
  const int kT = step_rows(waves);
  // rows before a segment start that the ring must hold: the band, the covered distances and
  // the rows of the queued slabs read at the first step (d - depth T back)
  int need = kMaxBand;
  for (int e = 0; e < a.n_cov; ++e) need = f.tab.dist[e] > need ? f.tab.dist[e] : need;
  if (n_q > 0) need = std::max(need, a.q_dist[0] - kT * kQDepth0);
  if (n_q > 1) need = std::max(need, a.q_dist[1] - kT * kQDepth1);
  a.warm = ((need + kT - 1) / kT) * kT;
  int early = kMaxBand;
  for (int e = 0; e < a.n_cov + n_q + n_far; ++e) early = f.tab.dist[e] > early ? f.tab.dist[e] : early;
  a.early_rows = early;
  // segments per head: see ring_segments
  const int64_t tiles = (f.N + kT - 1) / kT;
  const int64_t segs = ring_segments(f.BH, tiles);
  a.seg_len = (int)(((tiles + segs - 1) / segs) * kT);
  a.segs = (int)segs;
  const unsigned blocks = (unsigned)(segs * f.BH);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kD));
  a.rope = f.rope;
  a.n_far = n_far;
  a.heads_per_plan = f.heads_per_plan;
  if (f.plan != nullptr) {
    if (f.mode == 0) return launch_mode<0, 8, true>(a, n_far, blocks, f.stream);
    return launch_mode<1, 8, true>(a, n_far, blocks, f.stream);
  }
  if (n_q > 0) return launch_queued(a, f.mode, n_q, n_far, blocks, f.stream);
  if (f.mode == 0) return launch_mode<0, 8>(a, n_far, blocks, f.stream);
  return launch_mode<1, 8>(a, n_far, blocks, f.stream);
}

}  // namespace fib
