// Dense causal attention normaliser (LSE) on MFMA, and the dropped attention mass of the
// sparse pattern.
//
// The diagnostic is the attention-gap measure of "SSA: Sparse Sparse Attention" (arXiv
// 2511.20102, gist.science summary, 1. Problem definition, item 1): the softmax weight that
// full attention gives to keys the sparse mechanism does not select. Applied to the
// Fibonacci-offset pattern ("Depth-Staggered Fibonacci Spacing for Sparse Attention", Method
// > Architecture and attention mechanism; integer offsets), for query i:
//   dropped(i) = 1 - sum_{j in S_i} softmax_dense(i, j) = 1 - exp(LSE_sparse(i) - LSE_dense(i)),
// since both softmaxes share the logits <R_i q_i, R_j k_j> / sqrt(D) and LSE_sparse is the
// log-sum of the same exponentials over S_i (the sparse forward returns it).
//
// LSE_dense is a causal Q K^T contraction, so it runs on MFMA: a rotation pass writes
// bf16 copies of R_p q_p and R_p k_p (RoPE at each row's position, fp32 math, round to
// nearest even), then each workgroup streams 64-key tiles of K^ through LDS against 128
// queries held in registers. S^T = K^ Q^T blocks come from v_mfma_f32_16x16x32_bf16 (lane
// (n, g) holds keys 4g..4g+3 of a 16-key block for query n); every lane keeps an online
// log-sum-exp over the keys it holds, and the four lanes of a query merge once at the end.
#include "ring_common.h"

namespace fib {
namespace {

using namespace ring;

constexpr int kDT = 64;      // keys per LDS tile
constexpr int kDQ = 128;     // queries per workgroup: 4 waves x 2 groups of 16
constexpr int kDRow = 144;   // LDS row stride (128 bytes + 16 padding: 16 rows on distinct banks)

// out[h][p] = R_p x[h][p] in bf16 for two tensors (x0 -> out0, x1 -> out1) of BH heads x N
// rows. The cos/sin of a position do not depend on the head or the tensor, so a block takes
// 64 positions (four lanes each; lane c owns the RoPE pairs (8c + t, 32 + 8c + t), t < 8)
// and hpb heads (blockIdx.y), computes each position's angles once and applies them to both
// tensors of all its heads.
constexpr int64_t kRotHeads = 2;      // heads per block, unless the grid's y limit needs more
constexpr int64_t kMaxGridY = 65535;
template <typename T>
__global__ __launch_bounds__(256) void rotate_rows_kernel(const T* __restrict__ x0, bf16_t* __restrict__ out0,
                                                          const T* __restrict__ x1, bf16_t* __restrict__ out1,
                                                          int64_t BH, int64_t N, int64_t hpb, Rope rope) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pos = t >> 2;
  if (pos >= N) return;
  const int c = (int)(t & 3);
  float2 cs[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) cs[u] = rope_cs(pos, rope.rev[8 * c + u]);
  const int64_t h0 = (int64_t)blockIdx.y * hpb;
  const int64_t h1 = h0 + hpb < BH ? h0 + hpb : BH;
  for (int64_t h = h0; h < h1; ++h) {
    const int64_t r = h * N + pos;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const T* x = which == 0 ? x0 : x1;
      bf16_t* out = which == 0 ? out0 : out1;
      float lo[8], hi[8], rl[8], rh[8];
      Vec8<T>::load(x + r * kD + 8 * c, lo);
      Vec8<T>::load(x + r * kD + kHalf + 8 * c, hi);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        rl[u] = lo[u] * cs[u].x - hi[u] * cs[u].y;
        rh[u] = hi[u] * cs[u].x + lo[u] * cs[u].y;
      }
      Vec8<bf16_t>::store(out + r * kD + 8 * c, rl);
      Vec8<bf16_t>::store(out + r * kD + kHalf + 8 * c, rh);
    }
  }
}

__global__ __launch_bounds__(256) void dense_lse_kernel(const bf16_t* __restrict__ qr, const bf16_t* __restrict__ kr,
                                                        float* __restrict__ lse, int64_t N, int64_t BH, int qtiles,
                                                        float scale_log2) {
  __shared__ __align__(16) uint8_t tile[2][kDT * kDRow];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int l = tid & 63;
  const int n = l & 15;
  const int g = l >> 4;
  // the heaviest query tiles (most keys) first, so the last wave of blocks is short
  const int qt = qtiles - 1 - (int)(blockIdx.x / BH);
  const int64_t head = blockIdx.x % BH;
  const int64_t i0 = (int64_t)qt * kDQ;
  const bf16_t* Q = qr + head * N * kD;
  const bf16_t* K = kr + head * N * kD;

  // B operands: query i0 + 32 wave + 16 qg + n, dims 8g.. (k-block 0) and 32 + 8g.. (k-block 1)
  uint4 bq[2][2];
  int64_t qi[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    qi[qg] = i0 + 32 * wave + 16 * qg + n;
    const int64_t ic = qi[qg] < N ? qi[qg] : N - 1;
    bq[qg][0] = *reinterpret_cast<const uint4*>(Q + ic * kD + 8 * g);
    bq[qg][1] = *reinterpret_cast<const uint4*>(Q + ic * kD + kHalf + 8 * g);
  }
  float m[2] = {-1e30f, -1e30f}, sum[2] = {0.f, 0.f};  // log2-domain running max and sum

  const int64_t last_q = (i0 + kDQ < N ? i0 + kDQ : N) - 1;
  const int nt = (int)(last_q / kDT) + 1;  // key tiles 0..nt-1 hold every key j <= last_q
  // staging: thread tid moves 32 bytes of key row tid / 4 (rows past the end repeat row N - 1;
  // they lie after every query and are masked); the next tile is loaded into registers while
  // the current one is multiplied
  const int srow = tid >> 2, sch = tid & 3;
  uint8_t* const sdst = &tile[0][0] + srow * kDRow + 32 * sch;
  uint4 st0, st1;
  {
    const int64_t j = srow < N ? srow : N - 1;
    const uint4* src = reinterpret_cast<const uint4*>(K + j * kD) + 2 * sch;
    st0 = src[0];
    st1 = src[1];
    *reinterpret_cast<uint4*>(sdst) = st0;
    *reinterpret_cast<uint4*>(sdst + 16) = st1;
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) {
      int64_t j = (int64_t)(t + 1) * kDT + srow;
      j = j < N ? j : N - 1;
      const uint4* src = reinterpret_cast<const uint4*>(K + j * kD) + 2 * sch;
      st0 = src[0];
      st1 = src[1];
    }
    f4 acc[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      // A operand: key row 16 kb + n of the tile, dims 8g.. and 32 + 8g..
      const uint8_t* rp = tile[buf] + (16 * kb + n) * kDRow + 16 * g;
      const bf16x8 a0 = as_bf8(*reinterpret_cast<const uint4*>(rp));
      const bf16x8 a1 = as_bf8(*reinterpret_cast<const uint4*>(rp + 64));
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        f4 c = {0.f, 0.f, 0.f, 0.f};
        c = mfma32(a0, as_bf8(bq[qg][0]), c);
        acc[qg][kb] = mfma32(a1, as_bf8(bq[qg][1]), c);
      }
    }
    // the tile reaches past the block's first query: keys after the query are masked
    const bool diag = (int64_t)t * kDT + kDT - 1 > i0;
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      if (diag) {
        // key t kDT + c comes after the query when its tile offset c exceeds lim
        const int lim = (int)(qi[qg] - (int64_t)t * kDT);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[qg][kb][v] = 16 * kb + 4 * g + v > lim ? -INFINITY : acc[qg][kb][v];
      }
      // raw logits: the scale (> 0) is applied in the exponent, exp2(s * scale_log2 - m)
      float tmax = acc[qg][0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, acc[qg][kb][v]);
      const float mn = fmaxf(m[qg], tmax * scale_log2);
      float acc_s = sum[qg] * ex2(m[qg] - mn);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc_s += ex2(fmaf(acc[qg][kb][v], scale_log2, -mn));
      sum[qg] = acc_s;
      m[qg] = mn;
    }
    if (t + 1 < nt) {
      uint8_t* d = sdst + (buf ^ 1) * (kDT * kDRow);
      *reinterpret_cast<uint4*>(d) = st0;
      *reinterpret_cast<uint4*>(d + 16) = st1;
    }
    __syncthreads();
  }
  // merge the four lanes of each query
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const float M = quad_max(m[qg]);
    const float L = quad_add(sum[qg] * ex2(m[qg] - M));
    if (g == 0 && qi[qg] < N) lse[head * N + qi[qg]] = (M + log2f(L)) * 0.69314718055994530942f;
  }
}

__global__ __launch_bounds__(256) void dropped_mass_kernel(const float* __restrict__ lse_sparse,
                                                           const float* __restrict__ lse_dense,
                                                           float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 1.f - expf(lse_sparse[i] - lse_dense[i]);
}

}  // namespace

size_t dense_lse_workspace_bytes(int64_t BH, int64_t N) { return (size_t)2 * BH * N * kD * sizeof(bf16_t); }

hipError_t launch_dense_lse(const void* q, const void* k, float* lse, int64_t BH, int64_t N, int dtype,
                            const Rope& rope, void* workspace, hipStream_t s) {
  bf16_t* qr = static_cast<bf16_t*>(workspace);
  bf16_t* kr = qr + (size_t)BH * N * kD;
  // x: 64 positions per block; y: groups of hpb heads
  int64_t hpb = kRotHeads;
  if ((BH + hpb - 1) / hpb > kMaxGridY) hpb = (BH + kMaxGridY - 1) / kMaxGridY;
  const dim3 rgrid((unsigned)((N * 4 + 255) / 256), (unsigned)((BH + hpb - 1) / hpb));
  if (dtype == 0)
    rotate_rows_kernel<float><<<rgrid, 256, 0, s>>>((const float*)q, qr, (const float*)k, kr, BH, N, hpb, rope);
  else
    rotate_rows_kernel<bf16_t><<<rgrid, 256, 0, s>>>((const bf16_t*)q, qr, (const bf16_t*)k, kr, BH, N, hpb,
                                                     rope);
  const int qtiles = (int)((N + kDQ - 1) / kDQ);
  const float sl2 = (float)(1.4426950408889634 / sqrt((double)kD));
  dense_lse_kernel<<<(unsigned)(qtiles * BH), 256, 0, s>>>(qr, kr, lse, N, BH, qtiles, sl2);
  return hipGetLastError();
}

hipError_t launch_dropped_mass(const float* lse_sparse, const float* lse_dense, float* out, int64_t n,
                               hipStream_t s) {
  dropped_mass_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(lse_sparse, lse_dense, out, n);
  return hipGetLastError();
}

}  // namespace fib
