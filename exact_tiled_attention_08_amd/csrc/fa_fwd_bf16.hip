// Attention forward for bfloat16 Q/K/V on gfx950: bf16 MFMA, float32 accumulation.
//
// One workgroup owns BR = 32*NW query rows of one (b, h); each of its NW waves owns 32
// rows. K and V stream through LDS in tiles of BC keys (two stages), and each wave folds
// every tile into its running state with the online-softmax recurrence:
// "FlashAttention: Attention Is Limited by Memory, Not Math", section "How tiling and
// online softmax stay exact" (running max m and sum l; previous sums rescaled by
// exp(m_old - m_new) when the max rises; divide by l once at the end), and
// "Explain FlashAttention ...", section "Keep only the state needed for the final
// weighted average". Each query block is read once and every key/value block streams
// past it ("Flash Attention Optimization", section "Active recall", question 6 and its
// answer); the query tiles of all heads are independent workgroups ("FlashAttention 1, 2
// and 3": parallel over sequence length as well as batch and heads).
//
// Register layouts (v_mfma_f32_32x32x16_bf16, lane l, g = l / 32):
//   A operand (32 x 16): row l%32, k = 8g..8g+7      B operand (16 x 32): col l%32, same k
//   C (32 x 32):        col l%32, row 8*(i/4) + 4g + i%4 for element i = 0..15
// The kernel computes S^T = K Q^T, so each lane's accumulator column is ONE query row and
// its 16 elements are 16 keys: the row max and row sum are in-lane except for one swap
// between the two lane halves (v_permlane32_swap), and the S^T accumulator converts in
// place into the P^T operand of O^T = V^T P^T. Inside each 16-key step of the PV
// contraction lane half g carries keys {4g..4g+3, 8+4g..8+4g+3}; the V^T operand is read
// in exactly that key order with the LDS transpose read ds_read_b64_tr_b16, so V stays
// row-major in LDS.
//
// Memory path: K and V tiles go from global memory straight into LDS
// (global_load_lds_dwordx4: lane i of a wave writes 16 bytes at LDS base + 16*i), so no
// VGPRs stage them. Rows are stored unpadded with an XOR swizzle of their 16-byte chunks
// so that the fragment reads are free of bank conflicts. Key rows past Nk are clamped to
// row Nk-1 (finite data that the mask then zero-weights).
//
// Rescaling: the accumulator is rescaled only in tiles where some row of the wave raised
// its running max; in the other tiles alpha = 1 for every row and the multiply is skipped.
// The offset is always the exact running max, so the largest weight of a row is exactly
// 1 and survives the rounding of P to bfloat16 without error (an offset that lags the
// max would leave the dominant weight at 2^delta, rounded by up to 2^-9 of its size).
#include "fa_internal.h"

namespace fa {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void gbl_void;

template <int D, int BC, int NW>
struct Cfg {
  static constexpr int BR = 32 * NW;          // query rows per workgroup
  static constexpr int T = 64 * NW;           // threads per workgroup
  static constexpr int ROWB = D * 2;          // bytes per K or V row in LDS (unpadded)
  static constexpr int CHR = D / 8;           // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;     // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILEB;     // K tile then V tile
  static constexpr int LDS = 2 * STAGE;
  static constexpr int SLOTS = BC * CHR;      // 16-byte slots per tile
  static constexpr int LOADS = SLOTS / T;     // direct loads per thread per tensor per tile
  static constexpr int ROWSTEP = T / CHR;     // rows between a thread's successive slots
  static_assert(D % 32 == 0 && BC % 32 == 0 && CHR >= 8, "tile shape");
  static_assert(SLOTS % T == 0 && T % CHR == 0, "slots must split evenly over threads");
  static_assert(LDS <= 160 * 1024, "LDS budget of one CU");
};

// XOR swizzles of the 16-byte chunk position within a row (bijective per row). LDS has 64
// banks of 4 bytes; a 16-byte read is served 16 lanes at a time and an 8-byte read 32
// lanes at a time, so each such group must touch distinct banks:
//  - K reads (ds_read_b128): 16 lanes read 16 consecutive rows at one chunk.
//  - V transpose reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows at 4
//    consecutive chunks (both 8-byte halves of each).
// With 256-byte rows (d = 128) a row spans all banks, so rows must differ in chunk
// position; with 128-byte rows (d = 64) odd rows already sit in the upper 32 banks.
template <int CHR>
__device__ __forceinline__ int swz_k(int r, int c) {
  return CHR == 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}
template <int CHR>
__device__ __forceinline__ int swz_v(int r, int c) {
  return CHR == 16 ? (c ^ ((r & 3) << 2)) : (c ^ (((r >> 1) & 1) << 2));
}

__device__ __forceinline__ float wave_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, BC, NW>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
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

  // Direct-load slots of this thread: slot s = n*T + tid -> row s / CHR, chunk position
  // s % CHR; the chunk fetched is the one the swizzle stores at that position.
  const int lrow = tid / C::CHR;
  const int lpos = tid % C::CHR;
  uint32_t koff[C::LOADS], voff[C::LOADS];  // byte offsets within a tile of keys
#pragma unroll
  for (int n = 0; n < C::LOADS; ++n) {
    const int r = lrow + n * C::ROWSTEP;
    koff[n] = (uint32_t)(r * C::ROWB + 16 * swz_k<C::CHR>(r, lpos));
    voff[n] = (uint32_t)(r * C::ROWB + 16 * swz_v<C::CHR>(r, lpos));
  }
  auto issue_tile = [&](int t, int stage) {
    const int kv0 = t * BC;
    char* Ks = smem + stage * C::STAGE;
    char* Vs = Ks + C::TILEB;
    // uniform 64-bit tile base + 32-bit per-lane offset (the saddr + voffset load form)
    const char* kt = (const char*)kh + (size_t)kv0 * C::ROWB;
    const char* vt = (const char*)vh + (size_t)kv0 * C::ROWB;
    const bool tail = kv0 + BC > p.Nk;  // rows past Nk re-read row Nk-1 instead
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
      uint32_t ko = koff[n], vo = voff[n];
      if (tail) {
        const int r = lrow + n * C::ROWSTEP;
        const int back = max(0, kv0 + r - (p.Nk - 1)) * C::ROWB;
        ko -= back;
        vo -= back;
      }
      const int wave_slot = (n * C::T + 64 * w) * 16;  // wave-uniform LDS byte offset
      __builtin_amdgcn_global_load_lds((const gbl_void*)(kt + ko), (lds_void*)(Ks + wave_slot),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const gbl_void*)(vt + vo), (lds_void*)(Vs + wave_slot),
                                       16, 0, 0);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running offset of this lane's row, in log2 units (score * c)
  float l = 0.f;        // running sum over this lane's half of the keys

  // per-lane constants of the V^T transpose reads
  const int trG = (lane >> 4) & 1;  // which 16 of the 32 output dims
  const int trj = lane & 15;

  if (ntiles > 0) issue_tile(0, 0);

  for (int t = 0; t < ntiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // my slots of tile t have landed
    __syncthreads();  // everyone's have; everyone is done with tile t-1's stage
    if (t + 1 < ntiles) issue_tile(t + 1, (t + 1) & 1);
    const int kv0 = t * BC;
    if (kv0 >= wave_kv_end) continue;  // whole tile above the diagonal for this wave
    const char* Ks = smem + (t & 1) * C::STAGE;
    const char* Vs = Ks + C::TILEB;

    // S^T tile = K_j Q_i^T  (BC keys x 32 queries per wave)
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      s[kb] = f32x16{};
      const int r = 32 * kb + col;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 ka = *(const bf16x8*)(Ks + r * C::ROWB + swz_k<C::CHR>(r, 2 * kk + g) * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[kk], s[kb], 0, 0, 0);
      }
    }

    // Mask on absolute positions: only tiles that cross the key tail or the diagonal.
    const bool need_mask = (kv0 + BC > p.Nk) || (CAUSAL && kv0 + BC - 1 > wq0 + p.off);
    if (need_mask) {
      // key kv0 + 32kb + 8(i/4) + 4g + i%4 is visible iff its in-tile offset <= lim
      const int lim = (CAUSAL ? min(p.Nk - 1, qrow + p.off) : p.Nk - 1) - kv0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
    }

    // Online softmax; the rescale of O is skipped when no row of the wave raised its max.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = wave_half_max(mx) * p.c;  // tile row max, log2 units (-inf if masked)
    const bool raise = mt > m;
    if (__any(raise)) {
      // rows that raised: alpha = exp(m_old - m_new) (0 when m_old = -inf); others: 1
      const float alpha = raise ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
      m = raise ? mt : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    const float m_use = (m == -INFINITY) ? 0.f : m;  // nothing visible yet: weights are 0

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
    l += lsum;

    // O^T += V_j^T P^T; the V^T operand comes from two transpose reads per 16-key step.
#pragma unroll
    for (int kc = 0; kc < BC / 16; ++kc)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x4 half[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = 16 * kc + 8 * h + 4 * g + (trj >> 2);
          const int cbyte = 64 * db + 32 * trG + 8 * (trj & 3);
          const int addr = r * C::ROWB + swz_v<C::CHR>(r, cbyte >> 4) * 16 + (cbyte & 15);
          half[h] = __builtin_bit_cast(
              bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + addr)));
        }
        const bf16x8 va = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kc], oacc[db], 0, 0, 0);
      }
  }

  // Epilogue: divide by l once; LSE = ln2 * (m + log2 l). Empty row: O = 0, LSE = -inf.
  const float lt = wave_half_sum(l);
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

int fwd_bf16_block_rows(int) { return 32 * 4; }

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, 64, 4>(p, causal, s);
  return launch<64, 128, 4>(p, causal, s);
}

}  // namespace fa
