// Internal launch interface between the C ABI (fibattn_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fib_common.h"

namespace fib {

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
};

hipError_t launch_fwd_generic(const FwdArgs& a);
bool fwd_ring_supported(const FwdArgs& a);
hipError_t launch_fwd_ring(const FwdArgs& a);
hipError_t launch_index_set(int32_t* out, int64_t N, int W, const Table& tab, int64_t cols, hipStream_t s);
// one query per (batch, head) at position N - 1 of a K/V cache of N rows: q and o are
// [BH, D], k and v [BH, N, D], lse [BH]
hipError_t launch_decode(const FwdArgs& a);

size_t bwd_workspace_bytes(int64_t BH, int64_t N, int dtype, int mode);
hipError_t launch_bwd(const BwdArgs& a);
// query side of the backward on the LDS ring (bf16, W <= 16): dQ, Delta [BH * N], one
// d(alpha) partial per workgroup (bwdq_ring_blocks of them) and, in interpolated mode when ps
// is not null, each (query, table entry)'s softmax weight P and dS (one ps_pack word) in
// ps[(head * kMaxEnt + entry) * N + query]
bool bwdq_ring_supported(const BwdArgs& a);
int64_t bwdq_ring_blocks(const BwdArgs& a);
hipError_t launch_bwdq_ring(const BwdArgs& a, float* delta, float* part, uint32_t* ps);
// key side on the LDS ring (bf16, W <= 16): dK, dV from Delta; in interpolated mode also
// from the (P, dS) pairs ps that the ring query side stored (required there)
bool bwdk_ring_supported(const BwdArgs& a);
hipError_t launch_bwdk_ring(const BwdArgs& a, const float* delta, const uint32_t* ps);

}  // namespace fib
