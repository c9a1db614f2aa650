// Attention forward with 8-bit floating-point Q, K, V (OCP E4M3) on gfx950 FP8 MFMA.
//
// "FlashAttention: Attention Is Limited by Memory, Not Math", section "FlashAttention 1, 2
// and 3", names FP8 as one of FlashAttention-3's additions; the method is unchanged: the
// same online softmax over key tiles ("How tiling and online softmax stay exact") with
// both products on the 8-bit matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4, float32
// accumulation, twice the bfloat16 rate). Scaling policy (not on the pages):
//   - q, k, v hold E4M3 values; the real inputs are q * q_descale, k * k_descale,
//     v * v_descale (one float32 factor per tensor);
//   - scores: S = (q k^T) * (scale * q_descale * k_descale), float32;
//   - probabilities enter the PV product as E4M3(256 * exp2(s - m)): the exponent offset is
//     the exact running max less 8, so a row's largest weight is exactly 256 (exact in
//     E4M3) and every weight keeps the format's full relative precision down to 2^-14;
//     l sums the same float32 values, so O = v_descale * sum(P v) / l needs no correction;
//   - O and LSE are float32.
//
// Work split and schedule are those of fa_fwd_bf16.hip (256 rows per workgroup, two wave
// groups alternating a matrix phase and a vector phase, K/V tiles global -> LDS directly),
// with 128-key tiles and these operand layouts (lane l, g = l / 32):
//   S^T = K Q^T, one MFMA per 32 keys x 64 dims: A = 32 bytes of one key row (dims
//   64kk + 32g ..), B = the same 32 dims of this lane's query row; C as for bfloat16
//   (lane column = query, element i = key 8(i/4) + 4g + i%4).
//   O^T += V^T P^T, one MFMA per 32 dims x 64 keys: B = the 32 probabilities this lane holds
//   for two 32-key blocks (its S^T elements, in element order); A = V^T in exactly that key
//   order, gathered with four LDS transpose reads ds_read_b64_tr_b8 (within a group of 16
//   lanes, lane t receives byte t%8 of the 8-byte chunks that lanes 2j + (t%16)/8 address,
//   j = 0..7; each lane addresses the chunk of one key row that holds its group's dims).
// Both products use the same k order for A and B, which is all the instruction requires.
#include <utility>

#include "fa_internal.h"

namespace fa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int D = 128;
constexpr int BC = 128;              // keys per tile
constexpr int NW = 8;                // waves per workgroup: two groups of four
constexpr int BR = 32 * NW;          // query rows per workgroup
constexpr int T = 64 * NW;
constexpr int TL = T / 2;            // threads that load one tensor (one group)
constexpr int ROWB = D;              // bytes per K or V row
constexpr int CHR = D / 16;          // 16-byte chunks per row (8)
constexpr int TILEB = BC * ROWB;     // 16 KB
constexpr int LDS = 4 * TILEB;       // two K buffers, two V buffers

// Ticket counters of the dynamic tail (map_block_tail), zero at load and put back to zero
// by the last ticket of every launch.
__device__ unsigned g_tail_tickets[kTailSlots];
constexpr int LOADS = BC * CHR / TL; // direct loads per thread per tile (4)
constexpr int ROWSTEP = TL / CHR;    // 32
constexpr int NKB = BC / 32;         // 32-key blocks per tile (4)
constexpr int NDB = D / 32;          // 32-dim blocks of O (4)
constexpr int NKK = D / 64;          // 64-dim contraction steps of S (2)
constexpr int NKC = BC / 64;         // 64-key contraction steps of PV (2)
static_assert(BC * CHR % TL == 0 && ROWSTEP % 16 == 0, "tile split");

// Chunk swizzles of the 128-byte rows (two rows per 256-byte span of the 64 banks):
//  - K is read with ds_read_b128, 16 consecutive rows at one chunk per LDS cycle: rows of
//    equal parity must differ in chunk position -> a bijection on row bits 1..3;
//  - V is read with the transpose reads: per 32 lanes, rows {0..3, 8..11} (+16n) at two
//    adjacent chunks -> rows of equal parity must differ in chunk bits 1..2 (row bits 1, 3).
__device__ __forceinline__ int fk(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int fv(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }

__device__ __forceinline__ f32x16 mfma8(v8i a, v8i b, f32x16 c) {
  // E4M3 x E4M3 (format selectors 0), block scales 2^(127 - 127) = 1
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ float wave_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool CAUSAL>
__global__ __launch_bounds__(T, 2) void fwd_fp8_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loader = w < NW / 2;  // group 0 loads K tiles, group 1 V tiles
  const int g = lane >> 5;
  const int col = lane & 31;

  int bh, qt;
  if (p.tail.draws == 0) {
    map_block(blockIdx.x, gridDim.x, p.nqt, p.hpg, CAUSAL, bh, qt);
  } else {
    __shared__ int s_item;
    if (!map_block_tail(p.tail, &g_tail_tickets[p.tail_slot], &s_item, p.nqt, p.hpg, CAUSAL, bh, qt))
      return;  // the pool was empty: no item for this workgroup
  }
  const int Nq = p.Nq, Nk = p.Nk, off = p.off;
  const int q0 = qt * BR;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + col;

  const unsigned char* __restrict__ qh = (const unsigned char*)p.q + (size_t)bh * Nq * D;
  const unsigned char* __restrict__ kh = (const unsigned char*)p.k + (size_t)bh * Nk * D;
  const unsigned char* __restrict__ vh = (const unsigned char*)p.v + (size_t)bh * Nk * D;

  // Q row in VGPRs: 32 dims (64kk + 32g ..) per contraction step, the B operand of S^T.
  v8i qb[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qb[kk] = v8i{};
    if (qrow < Nq) {
      const uint4* src = (const uint4*)(qh + (size_t)qrow * D + 64 * kk + 32 * g);  // 16-byte aligned
      const uint4 lo = src[0], hi = src[1];
      qb[kk] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  }

  int kv_end = Nk;
  int wave_kv_end = (wq0 < Nq) ? Nk : 0;
  if (CAUSAL) {
    kv_end = min(Nk, min(q0 + BR, Nq) - 1 + off + 1);
    if (wq0 < Nq) wave_kv_end = min(Nk, min(wq0 + 31, Nq - 1) + off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // Direct loads: slot s = n*TL + (tid % TL) holds chunk position s % CHR of row s / CHR;
  // the chunk fetched is the one the tensor's swizzle stores there.
  const int lrow = (tid % TL) / CHR;
  const int lpos = tid % CHR;
  const uint32_t lchunk = 16u * (uint32_t)(lpos ^ (loader ? fk(lrow) : fv(lrow)));
  const unsigned char* const lbase = loader ? kh : vh;
  const int wg4 = w & 3;
  auto kbuf = [&](int i) -> char* { return smem + i * TILEB; };
  auto vbuf = [&](int i) -> char* { return smem + (2 + i) * TILEB; };
  // Whole tiles need no row clamp: one loop-invariant lane offset, the row step in the
  // scalar base and the slot in the LDS base (no vector instruction per load).
  const uint32_t loff = (uint32_t)(lrow * ROWB) + lchunk;
  auto issue = [&](int t, char* dst) {
    const int kv0 = t * BC;
    if (kv0 + BC <= Nk) {
      const uint32_t lds0 = (uint32_t)(uintptr_t)((lds_char*)(dst + 64 * wg4 * 16));
      [&]<int... N>(std::integer_sequence<int, N...>) {
        (dma16_at<N * TL * 16>(lbase + (size_t)(kv0 + N * ROWSTEP) * ROWB, loff, lds0), ...);
      }(std::make_integer_sequence<int, LOADS>{});
      return;
    }
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const uint32_t lds = (uint32_t)(uintptr_t)((lds_char*)(dst + (n * TL + 64 * wg4) * 16));
      const int row = min(lrow + n * ROWSTEP, Nk - 1 - kv0);  // rows past Nk repeat row Nk-1
      dma16(lbase + (size_t)kv0 * ROWB, (uint32_t)(row * ROWB) + lchunk, lds);
    }
  };

  // K fragment of key block kb and 64-dim step kk: 32 bytes of row 32kb + col.
  auto kfrag = [&](const char* Ks, int kb, int kk) {
    const int r = 32 * kb + col;
    const char* row = Ks + r * ROWB;
    const int c0 = 4 * kk + 2 * g;
    const uint4 lo = *(const uint4*)(row + 16 * (c0 ^ fk(r)));
    const uint4 hi = *(const uint4*)(row + 16 * ((c0 + 1) ^ fk(r)));
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  // V^T fragment of 64-key step kc and 32-dim block db: read r (0..3) gives this lane the
  // 8 keys 64kc + 32(r/2) + 16(r%2) + 8(u/4) + 4g + u%4, u = 0..7 (its P bytes 8r..8r+7),
  // at dim 32db + lane%32. Lane t16 of each group of 16 addresses key u = t16/2, dim half
  // t16%2 of the 16 dims of its group.
  const int grp = lane >> 4, t16 = lane & 15;
  auto vfrag = [&](const char* Vs, int kc, int db) {
    const int u = t16 >> 1, h = t16 & 1;
    const int chunk = 2 * db + (grp & 1);
    v2i part[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = 64 * kc + 32 * (r >> 1) + 16 * (r & 1) + 8 * (u >> 2) + 4 * g + (u & 3);
      const int addr = key * ROWB + 16 * (chunk ^ fv(key)) + 8 * h;
      part[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(Vs + addr));
    }
    return v8i{part[0][0], part[0][1], part[1][0], part[1][1], part[2][0], part[2][1], part[3][0], part[3][1]};
  };

  auto needs_mask = [&](int t) {
    const int kv0 = t * BC;
    return (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > wq0 + off) || (kv0 >= wave_kv_end);
  };
  auto mask_s = [&](int t, f32x16 (&s)[NKB]) {
    const int lim = (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - t * BC - 4 * g;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running max of this lane's row, log2 units
  float l = 0.f;        // running sum of 256 * exp2(s - m) over this lane's half of the keys

  // Online softmax of one tile into the E4M3 operand pb: 256 * exp2(s c - m), rounded to
  // nearest even; O rescaled (only when some row of the wave raised its max).
  auto softmax = [&](f32x16 (&s)[NKB], v8i (&pb)[NKC]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = wave_half_max(mx) * p.c;
    const bool raise = mt > m;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
    m = raise ? mt : m;
    const float m_off = ((m == -INFINITY) ? 0.f : m) - 8.f;  // weights scaled by 2^8
    float lsum = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        // dword wd of pb[kc]: bytes 4wd..4wd+3 = elements of block 2kc + wd/4
        const int kb = 2 * kc + (wd >> 2), i0 = 4 * (wd & 3);
        float e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i0 + u], p.c, -m_off));
          lsum += e[u];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
        pb[kc][wd] = word;
      }
    l = l * alpha + lsum;
    if (__any(raise)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    }
  };

  // Matrix phase: O^T += V^T P^T (NPV MFMAs), then S^T of the next tile (NS MFMAs); the A
  // fragment of MFMA f is read RING-1 MFMAs ahead.
  constexpr int NPV = NKC * NDB, NS = NKB * NKK, NF = NPV + NS, RING = 3;
  auto afrag = [&](const char* Vs, const char* Ks, int f) {
    return f < NPV ? vfrag(Vs, f / NDB, f % NDB) : kfrag(Ks, (f - NPV) % NKB, (f - NPV) / NKB);
  };
  auto matrix = [&]<bool WITH_S>(const char* Vs, const char* Ks, const v8i (&pb)[NKC], f32x16 (&s)[NKB]) {
    constexpr int NM = WITH_S ? NF : NPV;
    v8i fr[RING];
#pragma unroll
    for (int f = 0; f < RING - 1; ++f) fr[f] = afrag(Vs, Ks, f);
#pragma unroll
    for (int f = 0; f < NM; ++f) {
      const int fn = f + RING - 1;
      if (fn < NM) fr[fn % RING] = afrag(Vs, Ks, fn);
      __builtin_amdgcn_sched_barrier(0);
      if (f < NPV) {
        oacc[f % NDB] = mfma8(fr[f % RING], pb[f / NDB], oacc[f % NDB]);
      } else {
        const int g2 = f - NPV;
        s[g2 % NKB] = mfma8(fr[f % RING], qb[g2 / NKB], g2 < NKB ? f32x16{} : s[g2 % NKB]);
      }
    }
  };
  auto compute_s = [&](const char* Ks, f32x16 (&s)[NKB]) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma8(kfrag(Ks, kb, kk), qb[kk], kk == 0 ? f32x16{} : s[kb]);
  };

  // Prologue and steps: as in fa_fwd_bf16.hip (group 1 runs one phase behind group 0).
  // Group 0 loads K_{j+2} at the start of its matrix phase of step j, into the buffer of K_j;
  // group 1 loads V_{j+1} at the start of its matrix phase of step j, into the buffer of
  // V_{j-1} (both groups finished reading it at the barrier before), and waits for it before
  // its mid-step barrier. Issuing a tile's direct loads holds the issuing waves for a few
  // hundred cycles, and here the vector phase is the longer one, so no load is issued in it
  // (measured against group 1 loading V_{j+2} at the end of its vector phase: +6.7% at
  // N = 8192 and +5.2% at N = 30000, bitwise-identical results).
  v8i pb[NKC];
  f32x16 s[NKB];
  if (ntiles > 0) issue(0, loader ? kbuf(0) : vbuf(0));
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and tile 0 have landed
  // Q through an empty asm: otherwise a merged path that bypasses the wait above makes the
  // compiler wait for the Q loads (vmcnt(0), which includes the tile loads just issued)
  // inside every matrix phase.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qb[kk]));
  if (ntiles > 0) {
    wg_barrier();
    if (ntiles > 1 && loader) issue(1, kbuf(1));
    if (wave_kv_end > 0) {
      compute_s(kbuf(0), s);
      if (needs_mask(0)) mask_s(0, s);
      softmax(s, pb);
    }
    if (!loader) wg_barrier();
  }
  auto step = [&](int j, int cur) {
    if (loader) wait_loads();
    wg_barrier();
    if (loader && j + 2 < ntiles) issue(j + 2, kbuf(cur));
    if (!loader && j + 1 < ntiles) issue(j + 1, vbuf(cur ^ 1));  // V_{j+1}
    const bool active = j * BC < wave_kv_end;
    if (active) matrix.template operator()<true>(vbuf(cur), kbuf(cur ^ 1), pb, s);
    if (!loader) wait_loads();
    wg_barrier();
    if (active) {
      if (needs_mask(j + 1)) mask_s(j + 1, s);
      softmax(s, pb);
    }
  };
  auto last_step = [&](int j, int cur) {
    wg_barrier();
    if (j * BC < wave_kv_end) matrix.template operator()<false>(vbuf(cur), kbuf(cur ^ 1), pb, s);
    wg_barrier();
  };
  if (ntiles > 0) {
    const int last = ntiles - 1;
    for (int j = 0; j < last; j += 2) {
      step(j, 0);
      if (j + 1 < last) step(j + 1, 1);
    }
    if (last & 1)
      last_step(last, 1);
    else
      last_step(last, 0);
    if (loader) wg_barrier();
  }

  // Epilogue: O = v_descale * acc / l; LSE = ln2 * (m + log2 l - 8) (l holds 2^8-scaled sums).
  // O leaves through this wave's own 8 KB of LDS, 64 columns at a time, so that each store
  // writes whole 256-byte segments of 4 rows rather than 32 bytes of each of 32 rows (as in
  // the bfloat16 kernel; chunk c of row r at chunk position c ^ (r % 16), free of bank
  // conflicts), with non-temporal stores (+0.5% at N = 8192 for the staging, the hint
  // neutral here). Every wave has passed its last LDS read at the barrier above.
  const float lt = wave_half_sum(l);
  const float f = lt > 0.f ? p.vscale / lt : 0.f;
  constexpr int kStage = 32 * 64 * 4;  // one wave's area
  static_assert(NW * kStage <= LDS, "epilogue staging exceeds the LDS");
  char* const ot = smem + w * kStage;
  float* const oh = p.o + (size_t)bh * Nq * D;
#pragma unroll
  for (int hh = 0; hh < D / 64; ++hh) {
#pragma unroll
    for (int dbh = 0; dbh < 2; ++dbh)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int db = 2 * hh + dbh;
        f32x4 val;
        val[0] = oacc[db][4 * jj + 0] * f;
        val[1] = oacc[db][4 * jj + 1] * f;
        val[2] = oacc[db][4 * jj + 2] * f;
        val[3] = oacc[db][4 * jj + 3] * f;
        const int c = 8 * dbh + 2 * jj + g;  // columns 64 hh + 4c .. 64 hh + 4c + 3
        *(f32x4*)(ot + col * 256 + ((c ^ (col & 15)) << 4)) = val;
      }
    asm volatile("" ::: "memory");  // one wave's LDS accesses complete in issue order
    const int c = lane & 15;
    f32x4 rd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      rd[i] = *(const f32x4*)(ot + r * 256 + ((c ^ (r & 15)) << 4));
    }
    float* const obase = oh + (size_t)(wq0 + (lane >> 4)) * D + 64 * hh + 4 * c;
    if (wq0 + 32 <= Nq) {  // all 32 rows of the wave exist
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * D));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (wq0 + 4 * i + (lane >> 4) < Nq)
          __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * D));
    }
    asm volatile("" ::: "memory");
  }
  if (qrow < Nq && g == 0 && p.lse)
    p.lse[(size_t)bh * Nq + qrow] = lt > 0.f ? (m + __log2f(lt) - 8.f) * kLn2 : -INFINITY;
}

}  // namespace

int fwd_fp8_block_rows() { return BR; }

int fwd_fp8_key_tile() { return BC; }

hipError_t launch_fwd_fp8(const FwdParams& prm, bool causal, hipStream_t s) {
  FwdParams p = prm;
  const int total = p.tail.draws ? 8 * p.tail.s + p.tail.draws : p.BH * p.nqt;
  if (causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<true>), dim3(total), dim3(T), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<false>), dim3(total), dim3(T), 0, s, p);
  return hipGetLastError();
}

}  // namespace fa
