// Attention backward for float32 Q/K/V/dO on gfx950: float32 MFMA, no narrower rounding.
//
// The gradients of the bfloat16 backward (the same formulas: dV = P^T dO, dP = dO V^T,
// dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q with D_i = dO_i . O_i and
// P_ij = exp(scale q_i.k_j - LSE_i), probabilities recomputed from the saved LSE as
// "Flash Attention Optimization", section "Sizing a tile, and why the backward pass
// recomputes instead of storing", describes), computed with v_mfma_f32_32x32x2_f32 on
// float32 operands throughout: P and dS are never rounded below float32. This path exists
// for exact float32 gradients next to the float32 forward, not for throughput: tiles go
// through LDS in one stage, with a workgroup barrier on each side.
//
// MFMA layouts (v_mfma_f32_32x32x2_f32, lane l, g = l / 32): A (32 x 2) row l%32, k = g;
// B (2 x 32) col l%32, k = g; C (32 x 32) col l%32, row 8(i/4) + 4g + i%4 for element i.
// A k-step can pair any two contraction indices as long as A and B agree, so the second
// product of each kernel contracts over queries (or keys) in the order the first product's
// accumulator holds them: step s takes element s of every lane, i.e. index
// 8(s/4) + 4g + s%4 in lane half g, and the A operand is read from LDS at that index.
//
//   bwd_f32_pre_kernel:  per query row LSE in log2 units (+inf for rows that see no key and
//                        for padding rows) and D_i = dO_i . O_i, into the workspace.
//   bwd_f32_dkdv_kernel: one workgroup per 128 keys of one (b, h), 4 waves x 32 keys;
//                        K and V rows in VGPRs as B operands of S = Q K^T and dP = dO V^T
//                        (one key per lane column), dK^T and dV^T in float32
//                        accumulators; 32-query tiles of Q, dO and the statistics in LDS.
//   bwd_f32_dq_kernel:   one workgroup per 128 query rows, 4 waves x 32 rows; Q and dO
//                        rows in VGPRs, S^T = K Q^T and dP^T = V dO^T (one query per lane
//                        column), dQ^T accumulated over 32-key tiles of K and V in LDS.
//                        Recomputing S and dP keeps every output written once
//                        (deterministic, no atomics).
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kT = 256;   // threads per workgroup (4 waves)
constexpr int kTile = 32; // rows per LDS tile

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Workspace: LSE2 of every padded query row, then D of every padded query row.
__device__ __forceinline__ const float* ws_lse2(const BwdParams& p, int bh) {
  return p.ws + (size_t)bh * p.Nq_pad;
}
__device__ __forceinline__ const float* ws_dsum(const BwdParams& p, int bh) {
  return p.ws + (size_t)p.BH * p.Nq_pad + (size_t)bh * p.Nq_pad;
}

// One row per 16 lanes (8 floats each), reduced across the 16 lanes.
template <int D>
__global__ __launch_bounds__(kT) void bwd_f32_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kT / TPR;
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;  // over BH * Nq_pad
  const int part = tid % TPR;
  const long long total = (long long)p.BH * p.Nq_pad;
  const int bh = (int)(row / p.Nq_pad);
  const int i = (int)(row - (long long)bh * p.Nq_pad);
  float acc = 0.f;
  if (row < total && i < p.Nq) {
    const size_t e = ((size_t)bh * p.Nq + i) * D + 8 * part;
    const f32x4 d0 = *(const f32x4*)((const float*)p.dout + e);
    const f32x4 d1 = *(const f32x4*)((const float*)p.dout + e + 4);
    const f32x4 o0 = *(const f32x4*)(p.o + e);
    const f32x4 o1 = *(const f32x4*)(p.o + e + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_fmaf(d0[t], o0[t], __builtin_fmaf(d1[t], o1[t], acc));
  }
#pragma unroll
  for (int sh = TPR / 2; sh >= 1; sh >>= 1) acc += __shfl_xor(acc, sh);
  if (row < total && part == 0) {
    float l2 = INFINITY;  // padding rows and rows that see no key: every P comes out 0
    if (i < p.Nq) {
      const float lse = p.lse[(size_t)bh * p.Nq + i];
      if (lse != -INFINITY) l2 = lse * kLog2e;
    }
    p.ws[(size_t)bh * p.Nq_pad + i] = l2;
    p.ws[(size_t)p.BH * p.Nq_pad + (size_t)bh * p.Nq_pad + i] = i < p.Nq ? acc : 0.f;
  }
}

// Stage rows r0 .. r0+31 of a [N][D] float32 head into LDS (rows past N are zero).
template <int D, int PITCH>
__device__ __forceinline__ void stage_rows(float* dst, const float* src, int r0, int N, int tid) {
  for (int ch = tid; ch < kTile * D / 4; ch += kT) {
    const int r = ch / (D / 4), c4 = ch % (D / 4);
    f32x4 x = f32x4{};
    if (r0 + r < N) x = *(const f32x4*)(src + (size_t)(r0 + r) * D + 4 * c4);
    *(f32x4*)(dst + r * PITCH + 4 * c4) = x;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kT, 1) void bwd_f32_dkdv_kernel(BwdParams p) {
  constexpr int PITCH = D + 4;  // floats per LDS row: 4-float pad against bank conflicts
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) float Qs[kTile * PITCH];
  __shared__ __attribute__((aligned(16))) float Ds[kTile * PITCH];
  __shared__ float St[2][kTile];  // LSE2 and D of the tile's queries

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x / p.nkt;
  const int k0 = (blockIdx.x - bh * p.nkt) * kBwdKeyRows;
  const int wk0 = k0 + 32 * w;
  const int key = wk0 + col;

  const float* __restrict__ qh = (const float*)p.q + (size_t)bh * p.Nq * D;
  const float* __restrict__ doh = (const float*)p.dout + (size_t)bh * p.Nq * D;
  const float* __restrict__ kh = (const float*)p.k + (size_t)bh * p.Nk * D;
  const float* __restrict__ vh = (const float*)p.v + (size_t)bh * p.Nk * D;
  const float* lse2 = ws_lse2(p, bh);
  const float* dsum = ws_dsum(p, bh);

  // B operands: element (k = d, col = key) for every step of the d contraction
  float kr[D / 2], vr[D / 2];
#pragma unroll
  for (int st = 0; st < D / 2; ++st) {
    kr[st] = key < p.Nk ? kh[(size_t)key * D + 2 * st + g] : 0.f;
    vr[st] = key < p.Nk ? vh[(size_t)key * D + 2 * st + g] : 0.f;
  }
  f32x16 dk[NDB], dv[NDB];
  // The accumulators stay in the matrix registers (AGPRs) for the whole loop: the empty asm
  // here and at the top of every iteration keeps the compiler from parking them in VGPRs
  // at the loop edge and copying them across every tile.
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = dv[db] = f32x16{};
    asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
  }

  // queries that can see one of this workgroup's keys: i + off >= k0 when causal
  int q_first = 0;
  if (CAUSAL) q_first = max(0, k0 - p.off) / kTile * kTile;
  for (int q0 = q_first; q0 < p.Nq; q0 += kTile) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
    __syncthreads();  // the previous tile has been read
    stage_rows<D, PITCH>(Qs, qh, q0, p.Nq, tid);
    stage_rows<D, PITCH>(Ds, doh, q0, p.Nq, tid);
    if (tid < kTile) {
      const int i = q0 + tid;  // < Nq_pad: padding rows carry LSE2 = +inf, D = 0
      St[0][tid] = lse2[i];
      St[1][tid] = dsum[i];
    }
    __syncthreads();
    if (wk0 >= p.Nk) continue;
    if (CAUSAL && q0 + kTile - 1 + p.off < wk0) continue;  // no query here sees these keys

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 2; ++st) {
      s = mfma_f32(Qs[col * PITCH + 2 * st + g], kr[st], s);
      dp = mfma_f32(Ds[col * PITCH + 2 * st + g], vr[st], dp);
    }
    // element i: query q0 + 8(i/4) + 4g + i%4, key `key`
    float pe[16], ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qi = 8 * (i >> 2) + 4 * g + (i & 3);
      const int q = q0 + qi;
      const bool vis = key < p.Nk && (!CAUSAL || key <= q + p.off);
      pe[i] = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c, -St[0][qi])) : 0.f;
      ds[i] = pe[i] * (dp[i] - St[1][qi]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the tile's queries, in accumulator order
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int qi = 8 * (st >> 2) + 4 * g + (st & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = mfma_f32(Ds[qi * PITCH + 32 * db + col], pe[st], dv[db]);
        dk[db] = mfma_f32(Qs[qi * PITCH + 32 * db + col], ds[st], dk[db]);
      }
    }
  }

  // dK^T, dV^T: lane column = key, element i = dim 32db + 8(i/4) + 4g + i%4
  if (key < p.Nk) {
    float* dkr = p.dk + ((size_t)bh * p.Nk + key) * D;
    float* dvr = p.dv + ((size_t)bh * p.Nk + key) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dk[db][4 * j + e] * p.scale;
          b[e] = dv[db][4 * j + e];
        }
        *(f32x4*)(dkr + 32 * db + 8 * j + 4 * g) = a;
        *(f32x4*)(dvr + 32 * db + 8 * j + 4 * g) = b;
      }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kT, 1) void bwd_f32_dq_kernel(BwdParams p) {
  constexpr int PITCH = D + 4;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) float Ks[kTile * PITCH];
  __shared__ __attribute__((aligned(16))) float Vs[kTile * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, col = lane & 31;
  const int bh = blockIdx.x / p.nqt;
  const int q0 = (blockIdx.x - bh * p.nqt) * kBwdQueryRows;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + col;

  const float* __restrict__ qh = (const float*)p.q + (size_t)bh * p.Nq * D;
  const float* __restrict__ doh = (const float*)p.dout + (size_t)bh * p.Nq * D;
  const float* __restrict__ kh = (const float*)p.k + (size_t)bh * p.Nk * D;
  const float* __restrict__ vh = (const float*)p.v + (size_t)bh * p.Nk * D;

  // B operands: element (k = d, col = query)
  float qr[D / 2], dr[D / 2];
#pragma unroll
  for (int st = 0; st < D / 2; ++st) {
    qr[st] = qrow < p.Nq ? qh[(size_t)qrow * D + 2 * st + g] : 0.f;
    dr[st] = qrow < p.Nq ? doh[(size_t)qrow * D + 2 * st + g] : 0.f;
  }
  // qrow < Nq_pad always (the grid covers whole 128-row tiles)
  const float l2 = ws_lse2(p, bh)[qrow];
  const float dsm = ws_dsum(p, bh)[qrow];
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dq[db] = f32x16{};
    asm volatile("" : "+a"(dq[db]));  // kept in AGPRs across the loop, as in the dK/dV kernel
  }

  int kv_end = p.Nk;
  int wave_kv_end = wq0 < p.Nq ? p.Nk : 0;
  if (CAUSAL) {
    kv_end = min(p.Nk, min(q0 + kBwdQueryRows, p.Nq) - 1 + p.off + 1);
    if (wq0 < p.Nq) wave_kv_end = min(p.Nk, min(wq0 + 31, p.Nq - 1) + p.off + 1);
  }
  for (int k0 = 0; k0 < kv_end; k0 += kTile) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+a"(dq[db]));
    __syncthreads();
    stage_rows<D, PITCH>(Ks, kh, k0, p.Nk, tid);
    stage_rows<D, PITCH>(Vs, vh, k0, p.Nk, tid);
    __syncthreads();
    if (k0 >= wave_kv_end) continue;

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 2; ++st) {
      s = mfma_f32(Ks[col * PITCH + 2 * st + g], qr[st], s);
      dp = mfma_f32(Vs[col * PITCH + 2 * st + g], dr[st], dp);
    }
    // element i: key k0 + 8(i/4) + 4g + i%4, query qrow
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = k0 + 8 * (i >> 2) + 4 * g + (i & 3);
      const bool vis = kj < p.Nk && (!CAUSAL || kj <= qrow + p.off);
      const float pe = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.c, -l2)) : 0.f;
      ds[i] = pe * (dp[i] - dsm);
    }
    // dQ^T += K^T dS^T over the tile's keys, in accumulator order
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kj = 8 * (st >> 2) + 4 * g + (st & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = mfma_f32(Ks[kj * PITCH + 32 * db + col], ds[st], dq[db]);
    }
  }

  if (qrow < p.Nq) {
    float* dqr = p.dq + ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = dq[db][4 * j + e] * p.scale;
        *(f32x4*)(dqr + 32 * db + 8 * j + 4 * g) = a;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& prm, hipStream_t s) {
  BwdParams p = prm;
  const long long rows = (long long)p.BH * p.Nq_pad;
  const int pre_blocks = (int)((rows + (kT / (D / 8)) - 1) / (kT / (D / 8)));
  hipLaunchKernelGGL((bwd_f32_pre_kernel<D>), dim3(pre_blocks), dim3(kT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_f32_dkdv_kernel<D, CAUSAL>), dim3(p.BH * p.nkt), dim3(kT), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_f32_dq_kernel<D, CAUSAL>), dim3(p.BH * p.nqt), dim3(kT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace fa
