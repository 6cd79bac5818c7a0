// Internal launch interface between the C ABI (fibattn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fib_common.h"

namespace fib {

// ---- split of the offset table for the LDS-ring kernels --------------------------------
// A ring kernel of `waves` waves takes 16 * waves queries per step and keeps the last
// kRingRows rows in LDS, so it serves table entries up to kRingRows - 16 * waves from the
// ring ("covered", a prefix of the sorted table) and reads the rest ("far", up to distance
// N - 1) from global memory. RingSplit holds the per-entry arrays the ring kernels take;
// unused slots hold harmless in-bounds distances and zero weights.
constexpr int kRingRows = 512;
constexpr int kSplitCov = 16;  // covered slots
constexpr int kSplitFar = 4;   // far slots
constexpr int kBandRows = 16;  // window rows ahead of a 16-query block

struct RingSplit {
  int n_cov, n_far;
  int need;        // rows before a step that the ring must hold: max(16, largest covered distance)
  int early_rows;  // max(16, largest usable distance): steps below it need position checks
  int dist[kSplitCov];
  float w[kSplitCov];
  float f[kSplitCov];
  int far_dist[kSplitFar];
  float far_w[kSplitFar];
  float far_f[kSplitFar];
  int unc_dist[2 * kSplitFar];  // far distances (interpolated: c and c - 1 per entry)
};

__host__ __device__ inline int ring_reach(int waves) { return kRingRows - 16 * waves; }

// Fills s from table t for sequences of N rows (entries at distance >= N are unusable).
// Counts beyond the slots are left in n_cov / n_far for the caller to check.
__host__ __device__ inline void make_split(const Table& t, int64_t N, int waves, int mode, RingSplit* s) {
  int n = 0;
  while (n < t.n && (int64_t)t.dist[n] < N) ++n;
  const int reach = ring_reach(waves);
  int cov = 0;
  while (cov < n && t.dist[cov] <= reach) ++cov;
  s->n_cov = cov;
  s->n_far = n - cov;
  s->need = kBandRows;
  for (int e = 0; e < cov; ++e) s->need = t.dist[e] > s->need ? t.dist[e] : s->need;
  s->early_rows = kBandRows;
  for (int e = 0; e < n; ++e) s->early_rows = t.dist[e] > s->early_rows ? t.dist[e] : s->early_rows;
  for (int e = 0; e < kSplitCov; ++e) {
    const bool use = e < cov;
    s->dist[e] = use ? t.dist[e] : kBandRows;
    s->w[e] = use ? t.w[e] : 0.f;
    s->f[e] = use ? t.f[e] : 0.f;
  }
  for (int x = 0; x < kSplitFar; ++x) {
    const bool use = x < n - cov && cov + x < kMaxEnt;
    s->far_dist[x] = use ? t.dist[cov + x] : reach + 1;
    s->far_w[x] = use ? t.w[cov + x] : 0.f;
    s->far_f[x] = use ? t.f[cov + x] : 0.f;
  }
  for (int x = 0; x < kSplitFar; ++x) {
    if (mode == 1) {
      s->unc_dist[2 * x] = s->far_dist[x];
      s->unc_dist[2 * x + 1] = s->far_dist[x] - 1;
    } else {
      s->unc_dist[x] = s->far_dist[x];
      s->unc_dist[kSplitFar + x] = 0;
    }
  }
}

// ---- alpha in device memory ------------------------------------------------------------
// The alpha-dependent launch data, built on the device from *alpha by launch_dev_plan: the
// table and its ring splits for 8-wave and 4-wave kernels. Kernels launched for an alpha
// range read it from here instead of their arguments.
struct DevPlan {
  Table tab;
  RingSplit s8;
  RingSplit s4;
};
struct BaseList {
  int32_t v[kMaxEnt];
};
// Several layers in one call: layer l's tensors are the l-th [B, H, N, D] block of
// [L, B, H, N, D] inputs and its plan is plan[l]; the kernels take head h's plan from
// plan[h / heads_per_plan] (heads_per_plan = B * H).
constexpr int kMaxLayers = 256;
struct AlphaList {
  float v[kMaxLayers];
};
// Builds plans out[0..L-1]: from alpha[l] in device memory clamped into [lo, hi] (alpha not
// null), else from host[l] as given.
hipError_t launch_dev_plan(DevPlan* out, const float* alpha, const AlphaList& host, int L, float alpha_lo,
                           float alpha_hi, const BaseList& base, int n_base, int W, int mode, int64_t N,
                           hipStream_t s);
// Upper bounds, over alpha in [lo, hi], of the covered and far counts of make_split (host).
void range_counts(float lo, float hi, const int32_t* base, int n_base, int W, int mode, int64_t N, int waves,
                  int* n_cov, int* n_far);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH, N;
  int dtype, mode, W;
  Table tab;
  Rope rope;
  hipStream_t stream;
  // alpha in device memory (null: tab holds the table): the kernels read the table and its
  // splits from *plan; the launch picks kernel instances that fit every alpha in
  // [alpha_lo, alpha_hi] (base/n_base give the range bounds)
  const DevPlan* plan = nullptr;
  float alpha_lo = 0.f, alpha_hi = 0.f;
  const int32_t* base = nullptr;
  int n_base = 0;
  int heads_per_plan = 0x7fffffff;  // several layers: B * H (see AlphaList)
  int layers = 1;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dalpha;
  int64_t BH, N;
  int dtype, mode, W;
  Table tab;
  Rope rope;
  void* workspace;
  hipStream_t stream;
  const DevPlan* plan = nullptr;  // as in FwdArgs
  float alpha_lo = 0.f, alpha_hi = 0.f;
  const int32_t* base = nullptr;
  int n_base = 0;
  int heads_per_plan = 0x7fffffff;
  int layers = 1;  // dalpha holds one value per layer
  // interpolated bf16 calls: table entries the (P, dS) words of the workspace have room for
  // per query (an upper bound on the entry count of every layer of the call)
  int ps_slots = 0;
};

hipError_t launch_fwd_generic(const FwdArgs& a);
bool fwd_ring_supported(const FwdArgs& a);
// the kernel instance a launch would pick (-1: the general kernel); calls over several
// layers launch runs of consecutive layers whose instances agree
int fwd_instance_key(const FwdArgs& a);
int bwdq_instance_key(const BwdArgs& a);
int bwdk_instance_key(const BwdArgs& a);
hipError_t launch_fwd_ring(const FwdArgs& a);
hipError_t launch_index_set(int32_t* out, int64_t N, int W, const Table& tab, int64_t cols, hipStream_t s);
// one query per (batch, head) at position N - 1 of a K/V cache of N rows: q and o are
// [BH, D], k and v [BH, N, D], lse [BH]
hipError_t launch_decode(const FwdArgs& a);
// forward of small problems (at most kGatherMaxRows query rows) that the ring kernel does not
// take: the decode kernel's structure with 1-4 queries per block, all keys requested at once
constexpr int64_t kGatherMaxRows = 1 << 16;
bool fwd_gather_preferred(const FwdArgs& a);
hipError_t launch_fwd_gather(const FwdArgs& a);

// dense causal LSE (bf16 MFMA on rotated bf16 copies of q and k in the workspace) and the
// dropped mass 1 - exp(lse_sparse - lse_dense)
size_t dense_lse_workspace_bytes(int64_t BH, int64_t N);
hipError_t launch_dense_lse(const void* q, const void* k, float* lse, int64_t BH, int64_t N, int dtype,
                            const Rope& rope, void* workspace, hipStream_t s);
hipError_t launch_dropped_mass(const float* lse_sparse, const float* lse_dense, float* out, int64_t n,
                               hipStream_t s);

// ps_slots: (P, dS) words per query (interpolated bf16 calls; ps_entry_slots)
size_t bwd_workspace_bytes(int64_t BH, int64_t N, int dtype, int mode, int ps_slots);
// table entries of an interpolated call whose alphas are at most alpha_hi: the base entries
// with alpha_hi * f >= W (the kept set only grows with alpha)
int ps_entry_slots(float alpha_hi, const int32_t* base, int n_base, int W);
hipError_t launch_bwd(const BwdArgs& a);
// query side of the backward on the LDS ring (bf16, W <= 16): dQ, Delta [BH * N], one
// d(alpha) partial per workgroup (bwdq_ring_blocks of them) and, in interpolated mode, the
// rotated rows R_i q_i in qr and R_j k_j in kr ([BH][N][D] bf16, every row) and, when ps is
// not null, each (query, table entry)'s softmax weight P and dS (one ps_pack word) in
// ps[(head * a.ps_slots + entry) * N + query] (qr and kr are not used in integer mode)
bool bwdq_ring_supported(const BwdArgs& a);
int64_t bwdq_ring_blocks(const BwdArgs& a);
hipError_t launch_bwdq_ring(const BwdArgs& a, float* delta, float* part, uint32_t* ps, bf16_t* qr, bf16_t* kr);
// key side on the LDS ring (bf16, W <= 16): dK, dV from Delta; in interpolated mode also
// from the rotated rows qr, kr and the (P, dS) pairs ps that the ring query side stored
// (required there)
bool bwdk_ring_supported(const BwdArgs& a);
// Also writes dalpha (one value per layer) from the query side's dal_n partials per layer
hipError_t launch_bwdk_ring(const BwdArgs& a, const float* delta, const uint32_t* ps, const float* dal_part,
                            int64_t dal_n, const bf16_t* qr, const bf16_t* kr);

}  // namespace fib
