// Attention forward for bfloat16 Q/K/V on gfx950: bf16 MFMA, float32 accumulation.
//
// One workgroup owns BR = 32*NW query rows of one (b, h); each of its NW waves owns
// 32 rows. K and V stream through LDS in tiles of BC keys (double-buffered), and each
// wave folds every tile into its running state with the online-softmax recurrence:
// "FlashAttention: Attention Is Limited by Memory, Not Math", section "How tiling and
// online softmax stay exact" (running max m and sum l; previous sums rescaled by
// exp(m_old - m_new) when the max rises; divide by l once at the end), and
// "Explain FlashAttention ...", section "Keep only the state needed for the final
// weighted average". The loop order is the one that reads each query block once and
// streams all key/value blocks past it ("Flash Attention Optimization", section
// "Active recall", question 6 and its answer), with the query tiles of all heads as
// independent workgroups ("FlashAttention 1, 2 and 3": parallel over sequence length
// as well as batch and heads).
//
// Register layouts (v_mfma_f32_32x32x16_bf16, lane l, g = l / 32):
//   A operand (32 x 16): row l%32, k = 8g..8g+7      B operand (16 x 32): col l%32, same k
//   C (32 x 32):        col l%32, row 8*(i/4) + 4g + i%4 for element i = 0..15
// The kernel computes S^T = K Q^T, so each lane's accumulator column is ONE query row
// and its 16 elements are 16 keys: the row max and row sum are in-lane except for one
// exchange with lane l^32, and the S^T accumulator converts in place into the P^T
// operand of O^T = V^T P^T. The key order inside the PV contraction is permuted to
// match; V is written to LDS transposed in that same permuted key order.
#include "fa_internal.h"

namespace fa {
namespace {

template <int D, int BC, int NW>
struct Cfg {
  static constexpr int BR = 32 * NW;          // query rows per workgroup
  static constexpr int T = 64 * NW;           // threads per workgroup
  static constexpr int KPITCH = D * 2 + 16;   // bytes per K row in LDS (16 B pad: no bank conflicts)
  static constexpr int VPITCH = BC * 2 + 16;  // bytes per V^T row in LDS
  static constexpr int KBYTES = BC * KPITCH;
  static constexpr int VBYTES = D * VPITCH;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int KCHUNKS = BC * D / 8;        // 16-byte pieces of a K tile
  static constexpr int VUNITS = (BC / 4) * (D / 8); // 4-key x 8-dim pieces of a V tile
  static constexpr int KPER = (KCHUNKS + T - 1) / T;
  static constexpr int VPER = (VUNITS + T - 1) / T;
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
  static_assert(LDS <= 160 * 1024, "LDS budget of one CU");
};

__device__ __forceinline__ uint32_t lo16x2(uint32_t a, uint32_t b) {  // {a.lo, b.lo}
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {  // {a.hi, b.hi}
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, BC, NW>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 5;
  const int col = lane & 31;

  int bh, qt;
  map_block(blockIdx.x, gridDim.x, p.nqt, p.hpg, CAUSAL, bh, qt);
  const int q0 = qt * C::BR;
  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + col;   // this lane's query row

  const uint16_t* __restrict__ qh = (const uint16_t*)p.q + (size_t)bh * p.Nq * D;
  const uint16_t* __restrict__ kh = (const uint16_t*)p.k + (size_t)bh * p.Nk * D;
  const uint16_t* __restrict__ vh = (const uint16_t*)p.v + (size_t)bh * p.Nk * D;

  // Q tile stays in VGPRs for the whole key loop, as the B operand of S^T = K Q^T.
  bf16x8 qb[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (qrow < p.Nq)
      qb[kk] = *(const bf16x8*)(qh + (size_t)qrow * D + 16 * kk + 8 * g);
    else
      qb[kk] = bf16x8{};
  }

  // Key tiles this workgroup visits, and the key bound of this wave (causal).
  int kv_end = p.Nk;
  int wave_kv_end = (wq0 < p.Nq) ? p.Nk : 0;
  if (CAUSAL) {
    const int last_q = min(q0 + C::BR, p.Nq) - 1;
    kv_end = min(p.Nk, last_q + p.off + 1);
    if (wq0 < p.Nq) wave_kv_end = min(p.Nk, min(wq0 + 31, p.Nq - 1) + p.off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  uint4 kreg[C::KPER];
  uint4 vreg[C::VPER][4];

  auto load_tile = [&](int t) {
    const int kv0 = t * BC;
#pragma unroll
    for (int n = 0; n < C::KPER; ++n) {
      const int ch = tid + n * C::T;
      const int row = ch / (D / 8), cc = ch % (D / 8);
      const int key = kv0 + row;
      kreg[n] = (ch < C::KCHUNKS && key < p.Nk)
                    ? *(const uint4*)(kh + (size_t)key * D + 8 * cc)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < C::VPER; ++n) {
      const int u = tid + n * C::T;
      const int dc = u % (D / 8), kq = u / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kv0 + 4 * kq + r;
        vreg[n][r] = (u < C::VUNITS && key < p.Nk)
                         ? *(const uint4*)(vh + (size_t)key * D + 8 * dc)
                         : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int stage) {
    char* Ks = smem + stage * C::STAGE;
    char* Vs = Ks + C::KBYTES;
#pragma unroll
    for (int n = 0; n < C::KPER; ++n) {
      const int ch = tid + n * C::T;
      if (ch < C::KCHUNKS) {
        const int row = ch / (D / 8), cc = ch % (D / 8);
        *(uint4*)(Ks + row * C::KPITCH + cc * 16) = kreg[n];
      }
    }
#pragma unroll
    for (int n = 0; n < C::VPER; ++n) {
      const int u = tid + n * C::T;
      if (u < C::VUNITS) {
        const int dc = u % (D / 8), kq = u / (D / 8);
        // keys 4kq..4kq+3 = 16c + 8a + 4g' + r land at V^T columns 16c + 8g' + 4a + r
        const int pos = 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
        const uint4 x0 = vreg[n][0], x1 = vreg[n][1], x2 = vreg[n][2], x3 = vreg[n][3];
        const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w};
        const uint32_t a1[4] = {x1.x, x1.y, x1.z, x1.w};
        const uint32_t a2[4] = {x2.x, x2.y, x2.z, x2.w};
        const uint32_t a3[4] = {x3.x, x3.y, x3.z, x3.w};
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          uint2 ev, od;
          ev.x = lo16x2(a0[wd], a1[wd]);
          ev.y = lo16x2(a2[wd], a3[wd]);
          od.x = hi16x2(a0[wd], a1[wd]);
          od.y = hi16x2(a2[wd], a3[wd]);
          *(uint2*)(Vs + (8 * dc + 2 * wd) * C::VPITCH + pos * 2) = ev;
          *(uint2*)(Vs + (8 * dc + 2 * wd + 1) * C::VPITCH + pos * 2) = od;
        }
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running max of this lane's row, in units of log2 (score * c)
  float l = 0.f;        // running sum over this lane's half of the keys

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) load_tile(t + 1);
    const int kv0 = t * BC;
    if (kv0 < wave_kv_end) {
      const char* Ks = smem + (t & 1) * C::STAGE;
      const char* Vs = Ks + C::KBYTES;

      // S^T tile = K_j Q_i^T  (BC keys x 32 queries per wave)
      f32x16 s[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 ka = *(const bf16x8*)(Ks + (32 * kb + col) * C::KPITCH + (16 * kk + 8 * g) * 2);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], s[kb], 0, 0, 0);
        }
      }

      // Mask on absolute positions: only tiles that cross the key tail or the diagonal.
      const bool need_mask = (kv0 + BC > p.Nk) || (CAUSAL && kv0 + BC - 1 > wq0 + p.off);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Nk - 1, qrow + p.off) : p.Nk - 1;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > lim) s[kb][i] = -INFINITY;
          }
      }

      // Online softmax: new running max, rescale factor, exponentials.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx * p.c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // empty so far: any offset
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;

      bf16x8 pb[BC / 16];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], p.c, -m_use));
          lsum += e;
          pb[2 * kb + (i >> 3)][i & 7] = (__bf16)e;  // round to nearest even
        }
      l = l * alpha + lsum;

      // O^T = alpha * O^T + V_j^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 va = *(const bf16x8*)(Vs + (32 * db + col) * C::VPITCH + (16 * kc + 8 * g) * 2);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], oacc[db], 0, 0, 0);
        }
    }
    if (t + 1 < ntiles) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: divide by l once; LSE = ln2 * (m + log2 l). Empty row: O = 0, LSE = -inf.
  const float lt = l + __shfl_xor(l, 32);
  if (qrow < p.Nq) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* orow = p.o + ((size_t)bh * p.Nq + qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 val;
        val[0] = oacc[db][4 * j + 0] * inv;
        val[1] = oacc[db][4 * j + 1] * inv;
        val[2] = oacc[db][4 * j + 2] * inv;
        val[3] = oacc[db][4 * j + 3] * inv;
        *(f32x4*)(orow + 32 * db + 8 * j + 4 * g) = val;
      }
    if (g == 0 && p.lse)
      p.lse[(size_t)bh * p.Nq + qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, int BC, int NW>
hipError_t launch(const FwdParams& prm, bool causal, hipStream_t s) {
  FwdParams p = prm;
  const int total = p.BH * p.nqt;
  if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, true>), dim3(total), dim3(64 * NW), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, false>), dim3(total), dim3(64 * NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int fwd_bf16_block_rows(int d) { return d == 64 ? 32 * 4 : 32 * 4; }

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, 64, 4>(p, causal, s);
  return launch<64, 128, 4>(p, causal, s);
}

}  // namespace fa
