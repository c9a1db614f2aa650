// Internal declarations shared by the HIP kernels and the C-ABI layer of libfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Vector types used as MFMA operands and for 16-byte memory transactions.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMaxSplits = 1024;  // largest num_splits of the split-KV decode

// Arguments of the prefill kernels (one struct keeps the launch signature small).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;     // may be null
  int BH;         // B * H
  int Nq;
  int Nk;
  int off;        // Nk - Nq: absolute position of query row 0 for causal masking
  int nqt;        // number of query tiles per (b, h)
  int hpg;        // (b, h) pairs per XCD group for the block -> tile mapping
  float c;        // scale * log2(e): scores are exponentiated base 2
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;     // may be null
  float* ws_o;    // [BH][S][d] partial weighted sums
  float* ws_ml;   // [BH][S][2] partial (m, l), m in log2-scaled units
  int BH;
  int Nk;
  int S;          // number of splits
  int chunk;      // keys per split, ceil(Nk / S)
  float c;        // scale * log2(e)
};

// Launchers (defined next to their kernels). Each returns the hipError_t of the launch.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s);

// Query rows per workgroup of each prefill kernel (host needs it for the grid).
int fwd_bf16_block_rows(int d);
int fwd_f32_block_rows(int d);

// Block -> (b*H + h, query tile) mapping shared by the prefill kernels.
//
// Workgroups are handed to the 8 XCDs round-robin by block id, and each XCD has
// its own L2. The first 8*floor(total/8) blocks are renumbered so that XCD x
// receives one contiguous run of work items; inside a run, items walk a group of
// `hpg` heads query-tile by query-tile, so the query tiles of one head run
// together on one XCD and share its K/V in L2. For causal attention the query
// tiles are issued heaviest (most key tiles) first, which evens out the tail.
__device__ __forceinline__ void map_block(int L, int total, int nqt, int hpg, bool causal,
                                          int& bh, int& qt) {
  const int per = total >> 3;
  const int n = (L < (per << 3)) ? (L & 7) * per + (L >> 3) : L;
  const int span = hpg * nqt;
  const int grp = n / span;
  const int j = n - grp * span;
  const int qi = j / hpg;
  qt = causal ? (nqt - 1 - qi) : qi;
  bh = grp * hpg + (j - qi * hpg);
}

}  // namespace fa
