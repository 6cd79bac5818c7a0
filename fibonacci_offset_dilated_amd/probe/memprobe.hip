// Memory-delivery probe for the long-context forward's access pattern (a measurement aid, not
// part of the library; run through `python bench.py --memprobe`).
//
// It moves the forward ring kernel's rows without its arithmetic: each workgroup (8 waves,
// one per CU, held there by 150 KB of dynamic LDS as the ring is) sweeps one segment of one
// head in 128-row steps, 16 rows per wave. Per step each wave loads the Q, K and V rows of its
// 16 rows, plus, for each "far" distance d, the K and V rows 16 rows starting d back, and
// stores one O row per query. The next step's rows are requested before this step's are
// used (one-step prefetch, as in the kernel). The time of a variant is the floor that this
// pattern of loads puts under a kernel that issues them.
//
// Variants: the lane layout of the 16-byte pieces (A: lane (n, g) holds row n, bytes 16g and
// 64 + 16g, the MFMA operand layout the kernel uses; B: 8 lanes per row, one 128-byte line per
// 8 lanes), the far distances (the long-context table's 566, 915, 1480 vs distances inside the
// last three steps, whose rows this workgroup has just read), nontemporal loads and stores,
// and the segment count.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#define CHECK(x)                                                                         \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess) {                                                              \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
      exit(1);                                                                           \
    }                                                                                    \
  } while (0)

constexpr int kRowPieces = 8;  // 16-byte pieces per 64-dim bf16 row
constexpr int kStep = 128;     // rows per step (8 waves x 16)

struct Args {
  const uint4* q;
  const uint4* k;
  const uint4* v;
  uint4* o;
  int N, seg_len, segs;
  int d[4];
};

// the lane's two pieces of the 16-row block starting at rb: (row, piece) pairs
template <int LAY>
__device__ __forceinline__ void pieces(int rb, int l, int* r0, int* c0, int* r1, int* c1) {
  if (LAY == 0) {
    *r0 = rb + (l & 15);
    *c0 = l >> 4;
    *r1 = *r0;
    *c1 = 4 + (l >> 4);
  } else {
    *r0 = rb + (l >> 3);
    *c0 = l & 7;
    *r1 = rb + 8 + (l >> 3);
    *c1 = l & 7;
  }
}

// NF far distances; LS, LF: lane layouts of the streamed and the far rows; NT: nontemporal
template <int NF, int LS, int LF, int NT>
__global__ __launch_bounds__(512, 1) void probe_kernel(Args a) {
  extern __shared__ uint4 lds[];
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int head = blockIdx.x / a.segs, seg = blockIdx.x % a.segs;
  const int s0 = seg * a.seg_len;
  const int s1 = s0 + a.seg_len < a.N ? s0 + a.seg_len : a.N;
  const size_t ho = (size_t)head * a.N * kRowPieces;
  const uint4 *Q = a.q + ho, *K = a.k + ho, *V = a.v + ho;
  uint4* O = a.o + ho;
  uint4 cq[2], ck[2], cv[2], fk[NF > 0 ? NF : 1][2], fv[NF > 0 ? NF : 1][2];
  // rows are clamped into [0, N): every access stays inside the head
  auto at = [&](int r, int c) -> size_t {
    r = r < 0 ? 0 : (r >= a.N ? a.N - 1 : r);
    return (size_t)r * kRowPieces + c;
  };
  auto ld = [&](const uint4* p, size_t i) -> uint4 {
    if constexpr (NT) {
      typedef __attribute__((ext_vector_type(4))) unsigned int u4;
      const u4 t = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p + i));
      return make_uint4(t[0], t[1], t[2], t[3]);
    } else {
      return p[i];
    }
  };
  auto load_step = [&](int p0) {
    const int rb = p0 + 16 * wave;
    int r0, c0, r1, c1;
    pieces<LS>(rb, l, &r0, &c0, &r1, &c1);
    cq[0] = ld(Q, at(r0, c0));
    cq[1] = ld(Q, at(r1, c1));
    ck[0] = ld(K, at(r0, c0));
    ck[1] = ld(K, at(r1, c1));
    cv[0] = ld(V, at(r0, c0));
    cv[1] = ld(V, at(r1, c1));
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      pieces<LF>(rb - a.d[f], l, &r0, &c0, &r1, &c1);
      fk[f][0] = K[at(r0, c0)];
      fk[f][1] = K[at(r1, c1)];
      fv[f][0] = V[at(r0, c0)];
      fv[f][1] = V[at(r1, c1)];
    }
  };
  load_step(s0);
  for (int p0 = s0; p0 < s1; p0 += kStep) {
    // consume every loaded word (a few integer ops), so no load is dead
    uint4 x = cq[0];
    x.x ^= cq[1].x ^ ck[0].y ^ ck[1].z ^ cv[0].w ^ cv[1].x;
    x.y ^= ck[0].x ^ cv[1].y;
    x.z ^= ck[1].w ^ cv[0].z;
    x.w ^= cq[1].w;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      x.x ^= fk[f][0].x ^ fv[f][1].y;
      x.y ^= fk[f][1].z ^ fv[f][0].w;
      x.z += fk[f][0].w + fv[f][1].x;
      x.w += fk[f][1].y + fv[f][0].z;
    }
    __syncthreads();
    lds[tid] = x;  // (keeps the LDS allocation, and so one workgroup per CU)
    load_step(p0 + kStep < s1 ? p0 + kStep : p0);
    int r0, c0, r1, c1;
    pieces<0>(p0 + 16 * wave, l, &r0, &c0, &r1, &c1);
    if (r0 < s1) {
      if constexpr (NT) {
        typedef __attribute__((ext_vector_type(4))) unsigned int u4;
        const u4 t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<u4*>(O + at(r0, c0)));
        __builtin_nontemporal_store(t, reinterpret_cast<u4*>(O + at(r1, c1)));
      } else {
        O[at(r0, c0)] = x;
        O[at(r1, c1)] = x;
      }
    }
  }
}

template <int NF, int LS, int LF, int NT>
void run(const Args& a, const char* name) {
  const int smem = 150 * 1024;
  const int blocks = 32 * a.segs;
  CHECK(hipFuncSetAttribute((const void*)probe_kernel<NF, LS, LF, NT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            smem));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<float> ts;
  for (int it = 0; it < 13; ++it) {
    CHECK(hipEventRecord(e0));
    probe_kernel<NF, LS, LF, NT><<<blocks, 512, smem>>>(a);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (it >= 3) ts.push_back(ms);
  }
  std::sort(ts.begin(), ts.end());
  const float med = ts[ts.size() / 2];
  const double rows = 32.0 * a.N;
  const double moved = rows * (512.0 + NF * 256.0);  // Q, K, V read, O written, far K and V
  printf("{\"variant\": \"%s\", \"ms\": %.4f, \"moved_gb\": %.3f, \"moved_tbs\": %.3f, "
         "\"fwd_algorithmic_frac_of_8tbs\": %.4f}\n",
         name, med, moved / 1e9, moved / (med * 1e-3) / 1e12, rows * 516.0 / (med * 1e-3) / 8e12);
  fflush(stdout);
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
}

int main() {
  const int H = 32, N = 131072;  // the long-context shape, B = 1
  const size_t bytes = (size_t)H * N * kRowPieces * sizeof(uint4);
  uint4 *q, *k, *v, *o;
  CHECK(hipMalloc(&q, bytes));
  CHECK(hipMalloc(&k, bytes));
  CHECK(hipMalloc(&v, bytes));
  CHECK(hipMalloc(&o, bytes));
  CHECK(hipMemset(q, 1, bytes));
  CHECK(hipMemset(k, 2, bytes));
  CHECK(hipMemset(v, 3, bytes));
  CHECK(hipMemset(o, 0, bytes));
  Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.N = N;
  a.segs = 16;  // 512 workgroups of 8192 rows, as the forward kernel splits this shape
  a.seg_len = N / a.segs;
  a.d[0] = 566;
  a.d[1] = 915;
  a.d[2] = 1480;
  a.d[3] = 350;
  run<0, 0, 0, 0>(a, "stream A");
  run<0, 1, 1, 0>(a, "stream B");
  run<0, 0, 0, 1>(a, "stream A nontemporal");
  run<1, 0, 0, 0>(a, "stream A + far 566 A");
  run<2, 0, 0, 0>(a, "stream A + far 566,915 A");
  run<3, 0, 0, 0>(a, "stream A + far 566,915,1480 A");
  run<3, 0, 1, 0>(a, "stream A + far 566,915,1480 B");
  run<3, 1, 1, 0>(a, "stream B + far 566,915,1480 B");
  run<3, 0, 0, 1>(a, "stream A + far 566,915,1480 A nontemporal");
  a.d[0] = 130;
  a.d[1] = 260;
  a.d[2] = 350;
  run<3, 0, 0, 0>(a, "stream A + far 130,260,350 A");
  a.d[0] = 566;
  a.d[1] = 915;
  a.d[2] = 1480;
  a.segs = 32;
  a.seg_len = N / a.segs;
  run<3, 0, 0, 0>(a, "32 segments: stream A + far 566,915,1480 A");
  a.segs = 8;
  a.seg_len = N / a.segs;
  run<3, 0, 0, 0>(a, "8 segments: stream A + far 566,915,1480 A");
  CHECK(hipFree(q));
  CHECK(hipFree(k));
  CHECK(hipFree(v));
  CHECK(hipFree(o));
  return 0;
}
