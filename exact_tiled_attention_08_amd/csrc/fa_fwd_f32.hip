// Attention forward for float32 Q/K/V on gfx950: float32 MFMA, no narrower rounding.
//
// Same recurrence and work split as the bfloat16 kernel (running max m, running sum l,
// rescale by exp(m_old - m_new), divide once at the end: "FlashAttention: Attention Is
// Limited by Memory, Not Math", section "How tiling and online softmax stay exact"),
// with v_mfma_f32_32x32x2_f32. That instruction takes one k-value per lane
// (A: row l%32, k = l/32; B: col l%32, k = l/32; C as in the bf16 kernel), so V is read
// from LDS in its natural [key][d] layout and needs no transposition. Single-stage LDS:
// this path exists for exact float32 results, not for throughput.
//
// Additive bias (BIAS, float32 like the inputs): added to the scaled scores before the
// softmax ("Explain FlashAttention ...", section "Keep only the state needed for the final
// weighted average"); each lane reads the bias of its own query row and 16 keys per tile
// straight from global memory. Keys past Nk are not read.
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBC = 32;  // keys per tile
constexpr int kNW = 4;   // waves per workgroup (32 query rows each)

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(64 * kNW, 2) void fwd_f32_kernel(FwdParams p) {
  constexpr int PITCH = D + 4;  // floats per LDS row (4-float pad against bank conflicts)
  constexpr int T = 64 * kNW;
  constexpr int BR = 32 * kNW;
  __shared__ __attribute__((aligned(16))) float Ks[kBC * PITCH];
  __shared__ __attribute__((aligned(16))) float Vs[kBC * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, col = lane & 31;
  int bh, qt;
  map_block(blockIdx.x, gridDim.x, p.nqt, p.hpg, CAUSAL, bh, qt);
  const int q0 = qt * BR, wq0 = q0 + 32 * w, qrow = wq0 + col;

  const float* __restrict__ qh = (const float*)p.q + (size_t)bh * p.Nq * D;
  const float* __restrict__ kh = (const float*)p.k + (size_t)bh * p.Nk * D;
  const float* __restrict__ vh = (const float*)p.v + (size_t)bh * p.Nk * D;
  // bias row of this lane's query (clamped to Nq-1: rows past Nq are never stored)
  const float* brow = nullptr;
  if constexpr (BIAS) {
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    brow = (const float*)p.bias + (size_t)b * p.bsb + (size_t)h * p.bsh +
           (size_t)min(qrow, p.Nq - 1) * p.bsq;
  }
  const float cs = BIAS ? kLog2e : p.c;  // with a bias, scores arrive scaled (s * scale + bias)

  // Q^T operand: element (k = 2*step + g, col = query) for every step of the contraction.
  float qv[D / 2];
#pragma unroll
  for (int st = 0; st < D / 2; ++st) qv[st] = (qrow < p.Nq) ? qh[(size_t)qrow * D + 2 * st + g] : 0.f;

  int kv_end = p.Nk;
  int wave_kv_end = (wq0 < p.Nq) ? p.Nk : 0;
  if (CAUSAL) {
    const int last_q = min(q0 + BR, p.Nq) - 1;
    kv_end = min(p.Nk, last_q + p.off + 1);
    if (wq0 < p.Nq) wave_kv_end = min(p.Nk, min(wq0 + 31, p.Nq - 1) + p.off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + kBC - 1) / kBC : 0;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * kBC;
    // stage K_j and V_j (rows past Nk are zero)
    for (int ch = tid; ch < kBC * D / 4; ch += T) {
      const int row = ch / (D / 4), c4 = ch % (D / 4), key = kv0 + row;
      f32x4 kx = f32x4{}, vx = f32x4{};
      if (key < p.Nk) {
        kx = *(const f32x4*)(kh + (size_t)key * D + 4 * c4);
        vx = *(const f32x4*)(vh + (size_t)key * D + 4 * c4);
      }
      *(f32x4*)(Ks + row * PITCH + 4 * c4) = kx;
      *(f32x4*)(Vs + row * PITCH + 4 * c4) = vx;
    }
    __syncthreads();

    if (kv0 < wave_kv_end) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[col * PITCH + 2 * st + g], qv[st], s, 0, 0, 0);
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + 8 * (i >> 2) + 4 * g + (i & 3);
          const float bv = key < p.Nk ? brow[key] : 0.f;
          s[i] = __builtin_fmaf(s[i], p.scale, bv);
        }
      }

      const bool need_mask = (kv0 + kBC > p.Nk) || (CAUSAL && kv0 + kBC - 1 > wq0 + p.off);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Nk - 1, qrow + p.off) : p.Nk - 1;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kv0 + 8 * (i >> 2) + 4 * g + (i & 3) > lim) s[i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx * cs);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cs, -m_use));
        lsum += s[i];
      }
      l = l * alpha + lsum;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      // O^T += V^T P^T, one key per lane group per step: step i uses key 8(i/4)+4g+i%4
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * g + (i & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * PITCH + 32 * db + col], s[i], oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32);
  if (qrow < p.Nq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* orow = p.o + ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = oacc[db][4 * j + e] * inv;
        *(f32x4*)(orow + 32 * db + 8 * j + 4 * g) = val;
      }
    if (g == 0 && p.lse)
      p.lse[(size_t)bh * p.Nq + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, bool BIAS>
hipError_t launch(const FwdParams& prm, bool causal, hipStream_t s) {
  FwdParams p = prm;
  const int total = p.BH * p.nqt;
  if (causal)
    hipLaunchKernelGGL((fwd_f32_kernel<D, true, BIAS>), dim3(total), dim3(64 * kNW), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, false, BIAS>), dim3(total), dim3(64 * kNW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int fwd_f32_block_rows(int) { return 32 * kNW; }

hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s) {
  return d == 128 ? launch<128, false>(p, causal, s) : launch<64, false>(p, causal, s);
}

hipError_t launch_fwd_f32_bias(const FwdParams& p, int d, bool causal, hipStream_t s) {
  return d == 128 ? launch<128, true>(p, causal, s) : launch<64, true>(p, causal, s);
}

}  // namespace fa
