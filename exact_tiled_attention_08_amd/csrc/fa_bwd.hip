// Attention backward for bfloat16 Q/K/V/dO on gfx950: bf16 MFMA, float32 accumulation.
//
// Gradients of a loss L with respect to Q, K and V given dO = dL/dO, for the attention of
// fa_fwd. The probabilities are recomputed tile by tile from the saved per-row log-sum-exp
// instead of being stored ("Flash Attention Optimization", section "Sizing a tile, and why
// the backward pass recomputes instead of storing"; "Explain FlashAttention ...", section
// "Exact attention, finite precision and backward"). With P_ij = exp(scale q_i.k_j - LSE_i)
// (0 where masked), the chain rule through O = P V and the row softmax gives
//
//   dV_j = sum_i P_ij dO_i          dP_ij = dO_i . v_j          D_i = dO_i . O_i
//   dS_ij = P_ij (dP_ij - D_i)      dQ_i = scale sum_j dS_ij k_j    dK_j = scale sum_i dS_ij q_i
//
// (D_i = sum_j P_ij dP_ij because O_i = sum_j P_ij v_j.)
//
// Three launches on one stream:
//   1. bwd_pre_kernel: D_i and LSE_i in log2 units per query row, into the workspace.
//   2. bwd_dkdv_kernel: one workgroup per 128 keys of one (b, h); each of its 4 waves keeps
//      32 keys' K and V rows in VGPRs and their dK, dV in float32 accumulators while the
//      query tiles (Q, dO and the row statistics, 64 rows each) stream through LDS. Each
//      tile is one stream of MFMAs with the fragment reads prefetched and the float32 work
//      of one 32-query step spread between the MFMAs of the other step. On the few tiles
//      that cross the causal diagonal, masked pairs enter as S = -inf through the initial
//      accumulator of the S product (same stream, its own loop); the other tiles start it
//      from zero.
//   3. bwd_dq_kernel: one workgroup per 128 query rows of one (b, h); each wave keeps 32
//      rows' Q and dO in VGPRs and its dQ in float32 accumulators while 64-key K and V tiles
//      stream through LDS. It recomputes S and dP rather than adding partial dQ from the
//      dK/dV workgroups with atomics: every output element is written once, in a fixed
//      order, so the result is deterministic.
//
// The same three kernels serve packed batches of variable-length sequences (VARLEN): a
// pair's rows are then one sequence of one head in [total][H][d] tensors (pair_view), and
// workgroups whose tile lies past their sequence's end return before any barrier.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16, lane l, g = l / 32):
//   A (32 x 16): row l%32, k = 8g..8g+7      B (16 x 32): col l%32, same k
//   C (32 x 32): col l%32, row 8*(i/4) + 4g + i%4 for element i = 0..15
// dK/dV kernel: S = Q K^T and dP = dO V^T put one KEY per lane column (16 queries per
// lane), so S, P, dP and dS convert in place into the B operands of dV^T = dO^T P and
// dK^T = Q^T dS; the A operands dO^T and Q^T come from row-major LDS tiles through the
// transpose read ds_read_b64_tr_b16, in the query order of the B operand (lane half g holds
// queries {4g..4g+3, 8+4g..8+4g+3} of each 16-query step). The dQ kernel is the mirror
// image: S^T = K Q^T and dP^T = V dO^T put one QUERY per lane column and dQ^T = K^T dS^T
// reads K^T by transpose.
//
// Precision: P and dS are rounded to bfloat16 (nearest even) as MFMA operands; S, dP, the
// statistics and every accumulation are float32; outputs are float32.
#include <utility>

#include "fa_internal.h"

namespace fa {
namespace {

// Ticket counters of the dynamic tails (map_block_tail) of the dK/dV and dQ kernels, zero
// at load and put back to zero by the last ticket of every launch.
__device__ unsigned g_tail_tickets[kTailSlots];

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kT = 256;    // threads per workgroup of the two main kernels (4 waves)
constexpr int kRows = 64;  // rows per LDS tile: queries (dK/dV kernel), keys (dQ kernel)

template <int D>
struct BCfg {
  static constexpr int ROWB = 2 * D;                // bytes per bf16 row
  static constexpr int CHR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILEB = kRows * ROWB;        // bytes of one tile
  static constexpr int LOADS = kRows * CHR / kT;    // direct loads per thread per tile
  static constexpr int ROWSTEP = kT / CHR;          // rows between a thread's slots
  static_assert(kRows * CHR % kT == 0 && ROWSTEP % 16 == 0, "tile split");
};

// XOR swizzle of the 16-byte chunks of LDS row r: chunk c sits at chunk position
// c ^ bswz(r). Every tile is read in two patterns and both must be free of bank conflicts
// on the 64 banks of 4 bytes:
//  (a) ds_read_b128 of one chunk from 16 consecutive rows (16 lanes per LDS cycle):
//      bswz must be a bijection on the row bits that select the bank;
//  (b) ds_read_b64_tr_b16 of 4 consecutive chunks from 4 consecutive rows (32 lanes):
//      the chunk-group bits of bswz (bit 2 and up) must differ between those rows.
// d = 128 (256-byte rows span all banks): bswz = rotation of r's low four bits.
// d = 64 (128-byte rows, odd rows in the upper half of the banks): rotation of bits 1..3.
template <int CHR>
__device__ __forceinline__ int bswz(int r) {
  return CHR == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Pattern (a): 8 bf16 of chunk c of row r (an A operand row fragment).
template <int D>
__device__ __forceinline__ bf16x8 rfrag(const char* t, int r, int c) {
  return *(const bf16x8*)(t + r * (2 * D) + 16 * (c ^ bswz<D / 8>(r)));
}

// Pattern (b): the A operand (32 columns x 16 rows of the tile, transposed) for the 16-row
// step starting at row r0 and the 32-column block db: lane l gets column 32*db + l%32 at
// rows r0 + {4g..4g+3, 8+4g..8+4g+3}.
template <int D>
__device__ __forceinline__ bf16x8 tfrag(const char* t, int r0, int db, int lane) {
  const int g = lane >> 5, trG = (lane >> 4) & 1, trj = lane & 15;
  bf16x4 half[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = r0 + 8 * h + 4 * g + (trj >> 2);
    const int cbyte = 64 * db + 32 * trG + 8 * (trj & 3);
    const int addr = r * (2 * D) + 16 * ((cbyte >> 4) ^ bswz<D / 8>(r)) + (cbyte & 15);
    half[h] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + addr)));
  }
  return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)((const lds_char*)p);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Offset of the statistics of query row i inside one head's workspace block.
__device__ __forceinline__ int stat_index(int i) { return (i >> 6) * 128 + (i & 63); }

// The rows of pair bh. Dense: (b, h) of [B][H][N][d] tensors, row stride d. VARLEN: pair
// bh = h*B + b is sequence b of head h in the packed [total][H][d] tensors, row stride H*d,
// its row counts from the offsets (clamped into the tensors, then to the caps Nq and Nk of
// the launch: rows past a cap are not computed) and its causal offset from its own counts.
struct PairView {
  int Nq, Nk, off;
  long long qbase, kbase;  // element offset of row 0 on the query side and the key side
  int rs;                  // elements between consecutive rows
  long long lbase;         // index of row 0's LSE
};
template <int D, bool VARLEN>
__device__ __forceinline__ PairView pair_view(const BwdParams& p, int bh) {
  PairView v;
  if constexpr (VARLEN) {
    const int h = bh / p.B;
    const int b = bh - h * p.B;
    const int qs = min(max(p.cu_q[b], 0), p.total_q);
    const int ks = min(max(p.cu_k[b], 0), p.total_k);
    v.Nq = min(min(max(p.cu_q[b + 1], qs), p.total_q) - qs, p.Nq);
    v.Nk = min(min(max(p.cu_k[b + 1], ks), p.total_k) - ks, p.Nk);
    v.off = p.top_left ? 0 : v.Nk - v.Nq;
    v.qbase = ((long long)qs * p.H + h) * D;
    v.kbase = ((long long)ks * p.H + h) * D;
    v.rs = p.H * D;
    v.lbase = (long long)h * p.total_q + qs;
  } else {
    v.Nq = p.Nq;
    v.Nk = p.Nk;
    v.off = p.off;
    v.qbase = (long long)bh * p.Nq * D;
    v.kbase = (long long)bh * p.Nk * D;
    v.rs = D;
    v.lbase = (long long)bh * p.Nq;
  }
  return v;
}

// ---------------------------------------------------------------- row statistics

template <int D, bool VARLEN = false>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;         // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;     // rows per block
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;  // over BH * Nq_pad
  const int part = tid % TPR;
  const long long total = (long long)p.BH * p.Nq_pad;
  const int bh = (int)(row / p.Nq_pad);
  const int i = (int)(row - (long long)bh * p.Nq_pad);
  float acc = 0.f;
  float l2 = INFINITY;
  const PairView pv = pair_view<D, VARLEN>(p, row < total ? bh : 0);
  if (row < total && i < pv.Nq) {
    const size_t e = (size_t)(pv.qbase + (long long)i * pv.rs) + 8 * part;
    const bf16x8 dov = *(const bf16x8*)((const __bf16*)p.dout + e);
    const f32x4 o0 = *(const f32x4*)(p.o + e);
    const f32x4 o1 = *(const f32x4*)(p.o + e + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc = __builtin_fmaf((float)dov[t], o0[t], acc);
      acc = __builtin_fmaf((float)dov[4 + t], o1[t], acc);
    }
    const float L = p.lse[pv.lbase + i];
    l2 = (L == -INFINITY) ? INFINITY : L * kLog2e;
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, TPR);
  if (row < total && part == 0) {
    float* w = p.ws + (size_t)bh * p.Nq_pad * 2 + stat_index(i);
    w[0] = l2;
    w[64] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV

// BIAS: the scores carry the additive bias of fa_fwd_bias (S = scale QK^T + bias), staged
// per query tile as a [64 query][128 key] bfloat16 tile next to Q and dO, with the same
// 256-byte-row swizzle, and read per lane (one key, 16 queries per step) with the same
// transpose reads as Q^T. DBIAS: dS, the gradient of a full bias, is also written out.
template <int D, bool CAUSAL, bool BIAS = false, bool DBIAS = false, bool VARLEN = false>
__global__ __launch_bounds__(kT, 1) void bwd_dkdv_kernel(BwdParams p) {
  using C = BCfg<D>;
  constexpr int BTILE = kRows * 2 * kBwdKeyRows;             // bias tile, 256-byte rows
  constexpr int BOFF = 2 * C::TILEB + 512;                    // its offset inside a stage
  constexpr int STAGE = BOFF + (BIAS ? BTILE : 0);  // Q tile, dO tile, 64 LSE2 + 64 D, bias
  static_assert(!DBIAS || BIAS, "the bias gradient needs the biased scores");
  static_assert(!(BIAS && VARLEN), "the bias is offered for dense batches only");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int col = lane & 31;

  // Low key tiles see the most queries under the causal mask; ascending order issues them first.
  int bh, kt;
  // (not compiled into the biased instances: it costs them registers)
  if (VARLEN || BIAS || p.tail_kv.draws == 0) {
    map_block(blockIdx.x, gridDim.x, p.nkt, p.hpg_kv, false, bh, kt);
  } else {
    __shared__ int s_item;
    if (!map_block_tail(p.tail_kv, &g_tail_tickets[p.slot_kv], &s_item, p.nkt, p.hpg_kv, false, bh, kt))
      return;  // the pool was empty: no item for this workgroup
  }
  const int k0 = kt * kBwdKeyRows;
  const int kw0 = k0 + 32 * w;  // first key of this wave
  const int key = kw0 + col;    // this lane's key
  const PairView pv = pair_view<D, VARLEN>(p, bh);
  const int Nq = pv.Nq, Nk = pv.Nk, off = pv.off, rs = pv.rs;
  if (VARLEN && k0 >= Nk) return;  // the whole workgroup: this sequence has no such keys

  const __bf16* __restrict__ qh = (const __bf16*)p.q + pv.qbase;
  const __bf16* __restrict__ doh = (const __bf16*)p.dout + pv.qbase;
  const __bf16* __restrict__ kh = (const __bf16*)p.k + pv.kbase;
  const __bf16* __restrict__ vh = (const __bf16*)p.v + pv.kbase;
  const float* __restrict__ wsh = p.ws + (size_t)bh * p.Nq_pad * 2;
  // bias of (b, h), query 0, key k0 (BIAS only)
  const uint16_t* biasw = nullptr;
  if constexpr (BIAS) {
    const int b = bh / p.H;
    biasw = (const uint16_t*)p.bias + (size_t)b * p.bsb + (size_t)(bh - b * p.H) * p.bsh + k0;
  }

  // K and V rows of this lane's key: the B operands of S = Q K^T and dP = dO V^T. Keys past
  // Nk are zero; their columns are independent of every other column and are not stored.
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (key < Nk) {
      kf[kk] = *(const bf16x8*)(kh + (size_t)key * rs + 16 * kk + 8 * g);
      vf[kk] = *(const bf16x8*)(vh + (size_t)key * rs + 16 * kk + 8 * g);
    } else {
      kf[kk] = bf16x8{};
      vf[kk] = bf16x8{};
    }
  }

  // Query tiles to visit: under the causal mask query i sees key j iff j <= i + off, so
  // the first query that sees key k0 is k0 - off.
  const int q_begin = CAUSAL ? max(0, k0 - off) : 0;
  const int t0 = q_begin / kRows;
  const int t1 = (Nq + kRows - 1) / kRows;

  // Direct loads: slot s = n*kT + tid holds chunk position s % CHR of tile row s / CHR; the
  // swizzle depends only on row bits that repeat every ROWSTEP rows.
  const int lrow = tid / C::CHR;
  const uint32_t lchunk = 16u * (uint32_t)((tid % C::CHR) ^ bswz<C::CHR>(lrow));
  auto stage = [&](int i) -> char* { return smem + i * STAGE; };
  auto issue = [&](int t, char* st) {
    const int r0 = t * kRows;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
      const int row = min(lrow + n * C::ROWSTEP, Nq - 1 - r0);  // rows past Nq repeat row Nq-1
      const uint32_t loff = (uint32_t)(row * rs * 2) + lchunk;
      const uint32_t dst = (uint32_t)((n * kT + 64 * w) * 16);
      dma16(qh + (size_t)r0 * rs, loff, lds_addr(st + dst));
      dma16(doh + (size_t)r0 * rs, loff, lds_addr(st + C::TILEB + dst));
    }
    if constexpr (BIAS) {
      // 64 rows x 16 chunks: slot n*kT + tid is row tid/16 + 16n at chunk position tid%16,
      // holding chunk (position ^ swizzle); rows past Nq repeat row Nq-1 and chunks at or
      // past Nk the chunk of key Nk-1 (their pairs are masked or not stored)
      const int brow = tid >> 4;
      const int bch = min((tid & 15) ^ bswz<16>(brow), (Nk - 1 - k0) >> 3);
      const char* base = (const char*)(biasw + (size_t)r0 * p.bsq);
      const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(st + BOFF + 64 * w * 16));
      [&]<int... N>(std::integer_sequence<int, N...>) {
        ((dma16(base, (uint32_t)(((long long)min(brow + 16 * N, Nq - 1 - r0) * p.bsq + 8 * bch) * 2),
                lbase + N * kT * 16)), ...);
      }(std::make_integer_sequence<int, BTILE / (16 * kT)>{});
    }
    // 512 bytes of statistics: lanes 0..15 the LSE2 values, 16..31 the D values
    if (w == 0 && lane < 32) dma16(wsh + (size_t)t * 128, 16u * lane, lds_addr(st + 2 * C::TILEB));
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
    // The accumulators live in the matrix registers (AGPRs) from here to the end of the
    // loops; without this and the pin after every tile the compiler keeps them in VGPRs at
    // the loop edge and copies all 128 of them out and back in every tile.
    asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
  }

  // One 64-query tile as a single stream of 4*NG MFMAs (NG = D/8 per group):
  //   group 0: S and dP of query step 0 (A = Q and dO rows), alternating
  //   group 1: S and dP of query step 1
  //   group 2: dV^T += dO^T P and dK^T += Q^T dS of step 0 (A = transposed reads), alternating
  //   group 3: the same for step 1
  // The A fragment of MFMA f is read from LDS RING-1 MFMAs ahead. The float32 work of step 0
  // (P = exp2(S c - LSE2), dS = P (dP - D), rounding to bfloat16) is spread over group 1's
  // MFMAs and that of step 1 over group 2's, so the matrix core and the vector ALU of the
  // SIMD work at the same time.
  auto tile_stream = [&](auto maskedc, const char* Qs, const char* dOs, const float* sts,
                         const f32x16 (&sinit)[2], const char* Bs, int qa0) {
    constexpr bool MASKED = decltype(maskedc)::value;
    constexpr int NG = D / 8, NF = 4 * NG, RING = 6, EPM = 16 / NG;  // elements per MFMA
    f32x16 s[2], dp[2];
    bf16x8 pb[2][2], dsb[2][2];
    // bias of element e of step x (query 32x + 8(e/4) + 4g + e%4, this lane's key): two
    // transpose reads per step from the [query][key] tile
    bf16x8 bb[2][2];
    if constexpr (BIAS) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int h = 0; h < 2; ++h) bb[x][h] = tfrag<kBwdKeyRows>(Bs, 32 * x + 16 * h, w, lane);
    }
    f32x4 L[2], Dv[2];  // LSE2 and D of one group of 4 elements, double-buffered
    bf16x8 fr[RING];
    auto frag = [&](auto fc) -> bf16x8 {
      constexpr int f = decltype(fc)::value, x = (f / NG) & 1, i = f % NG;
      if constexpr (f < 2 * NG) {
        return rfrag<D>((i & 1) ? dOs : Qs, 32 * x + col, 2 * (i >> 1) + g);
      } else {
        constexpr int st = i / (NG / 2), db = (i % (NG / 2)) >> 1;
        return tfrag<D>((i & 1) ? Qs : dOs, 32 * x + 16 * st, db, lane);
      }
    };
    // statistics of elements 4j..4j+3 of step x (queries 32x + 8j + 4g + 0..3)
    auto stats = [&](int x, int j) {
      L[j & 1] = *(const f32x4*)(sts + 32 * x + 8 * j + 4 * g);
      Dv[j & 1] = *(const f32x4*)(sts + 64 + 32 * x + 8 * j + 4 * g);
    };
    // The float32 work of one element is split over two MFMA slots: the exponential and
    // dP - D in one, the product and the bfloat16 roundings in the next, so that no
    // instruction waits for the exponential it follows.
    float pe_t[2][EPM], sd_t[2][EPM];
    auto front = [&](auto xc, auto ec, auto bc) {
      constexpr int x = decltype(xc)::value, e = decltype(ec)::value, b = decltype(bc)::value;
      if constexpr (BIAS) {  // (s * scale + bias) in log2 units
        const float sb = __builtin_fmaf(s[x][e], p.scale, (float)bb[x][e >> 3][e & 7]);
        pe_t[b][e % EPM] = __builtin_amdgcn_exp2f(__builtin_fmaf(sb, kLog2e, -L[(e >> 2) & 1][e & 3]));
      } else {
        pe_t[b][e % EPM] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[x][e], p.c, -L[(e >> 2) & 1][e & 3]));
      }
      sd_t[b][e % EPM] = dp[x][e] - Dv[(e >> 2) & 1][e & 3];
    };
    auto back = [&](auto xc, auto ec, auto bc) {
      constexpr int x = decltype(xc)::value, e = decltype(ec)::value, b = decltype(bc)::value;
      const float pe = pe_t[b][e % EPM];
      pb[x][e >> 3][e & 7] = (__bf16)pe;
      if constexpr (DBIAS) {
        const float ds = pe * sd_t[b][e % EPM];
        dsb[x][e >> 3][e & 7] = (__bf16)ds;
        const int qi = qa0 + 32 * x + 8 * (e >> 2) + 4 * g + (e & 3);
        if (qi < Nq && key < Nk) p.dbias[((size_t)bh * Nq + qi) * Nk + key] = ds;
      } else {
        dsb[x][e >> 3][e & 7] = (__bf16)(pe * sd_t[b][e % EPM]);
      }
    };
    auto step = [&](auto fc) {
      constexpr int f = decltype(fc)::value, grp = f / NG, i = f % NG;
      if constexpr (f + RING - 1 < NF) fr[(f + RING - 1) % RING] = frag(std::integral_constant<int, f + RING - 1>{});
      // statistics one group of 4 elements ahead of the element work (MPG MFMAs per group)
      constexpr int MPG = 4 / EPM;
      if constexpr (f == NG - MPG) stats(0, 0);
      if constexpr ((grp == 1 || grp == 2) && i % MPG == 0 && i / MPG + 1 < 4) stats(grp - 1, i / MPG + 1);
      if constexpr (f == 2 * NG - MPG) stats(1, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this MFMA
      if constexpr (grp < 2) {
        constexpr int kk = i >> 1;
        if constexpr (i & 1)
          dp[grp] = mfma(fr[f % RING], vf[kk], kk == 0 ? f32x16{} : dp[grp]);
        else
          s[grp] = mfma(fr[f % RING], kf[kk], kk == 0 ? (MASKED ? sinit[grp] : f32x16{}) : s[grp]);
      } else {
        constexpr int x = grp - 2, st = i / (NG / 2), db = (i % (NG / 2)) >> 1;
        if constexpr (i & 1)
          dk[db] = mfma(fr[f % RING], dsb[x][st], dk[db]);
        else
          dv[db] = mfma(fr[f % RING], pb[x][st], dv[db]);
      }
      if constexpr (grp == 1 || grp == 2) {
        [&]<int... E>(std::integer_sequence<int, E...>) {
          (front(std::integral_constant<int, grp - 1>{}, std::integral_constant<int, EPM * i + E>{},
                 std::integral_constant<int, i & 1>{}), ...);
          if constexpr (i > 0)
            (back(std::integral_constant<int, grp - 1>{}, std::integral_constant<int, EPM * (i - 1) + E>{},
                  std::integral_constant<int, (i - 1) & 1>{}), ...);
        }(std::make_integer_sequence<int, EPM>{});
      }
      if constexpr ((grp == 2 || grp == 3) && i == 0) {
        [&]<int... E>(std::integer_sequence<int, E...>) {
          (back(std::integral_constant<int, grp - 2>{}, std::integral_constant<int, EPM * (NG - 1) + E>{},
                std::integral_constant<int, (NG - 1) & 1>{}), ...);
        }(std::make_integer_sequence<int, EPM>{});
      }
    };
    [&]<int... F>(std::integer_sequence<int, F...>) {
      ((fr[F] = frag(std::integral_constant<int, F>{})), ...);
    }(std::make_integer_sequence<int, RING - 1>{});
    [&]<int... F>(std::integer_sequence<int, F...>) {
      (step(std::integral_constant<int, F>{}), ...);
    }(std::make_integer_sequence<int, NF>{});
  };

  // dS = 0 for query rows [r_begin, r_end) and this wave's 32 keys (pairs the causal mask
  // hides in tiles that are not visited): 8 rows of 32 keys per store of the wave, 4 keys
  // per lane.
  auto zero_dbias = [&](int r_begin, int r_end) {
    const int kq = kw0 + 4 * (lane & 7);
    for (int r = r_begin + (lane >> 3); r < r_end; r += 8) {
      float* row = p.dbias + ((size_t)bh * Nq + r) * Nk;
      if (kq + 3 < Nk && ((Nk & 3) == 0)) {
        *(f32x4*)(row + kq) = f32x4{};
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (kq + u < Nk) row[kq + u] = 0.f;
      }
    }
  };

  // Tiles before tm hold a query that misses a key of this workgroup (causal): they take
  // the masked stream; from tm on every pair is visible and the stream has no mask.
  const int tm = CAUSAL ? min(t1, max(t0, (k0 + kBwdKeyRows - 1 - off + kRows - 1) / kRows)) : t0;
  auto body = [&](int t, auto maskedc) {
    constexpr bool MASKED = decltype(maskedc)::value;
    const int cur = (t - t0) & 1;
    wait_loads();  // tile t (the only loads in flight)
    wg_barrier();  // tile t visible to all; everyone is done with the other stage
    if (t + 1 < t1) issue(t + 1, stage(cur ^ 1));
    const char* Qs = stage(cur);
    const char* dOs = Qs + C::TILEB;
    const float* sts = (const float*)(Qs + 2 * C::TILEB);
    const int qa0 = t * kRows;
    f32x16 sinit[2] = {f32x16{}, f32x16{}};
    if constexpr (MASKED) {
      // no query of this tile sees a key of this wave: nothing to add (dS = 0 there)
      if (qa0 + kRows - 1 + off < kw0) {
        if constexpr (DBIAS) zero_dbias(qa0, min(qa0 + kRows, Nq));
        return;
      }
      // Masked pairs enter as S = -inf through the initial accumulator of the S product, so
      // that P = exp2(-inf) = 0 and dS = 0 with no extra work in the stream; element e of
      // step x is query qa0 + 32x + 8(e/4) + 4g + e%4 and is masked iff key > query + off.
      // Query rows past Nq need no mask: their LSE2 is +inf.
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int lim = key - off - qa0 - 32 * x - 4 * g;  // visible iff 8(e/4) + e%4 >= lim
#pragma unroll
        for (int e = 0; e < 16; ++e) sinit[x][e] = (8 * (e >> 2) + (e & 3) < lim) ? -INFINITY : 0.f;
      }
    }
    tile_stream(maskedc, Qs, dOs, sts, sinit, Qs + BOFF, qa0);
  };
  auto pin = [](f32x16 (&a)[D / 32], f32x16 (&b)[D / 32]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) asm volatile("" : "+a"(a[db]), "+a"(b[db]));
  };

  if (t0 < t1) issue(t0, stage(0));
  // The K and V rows must have landed before the loop, and the compiler must not wait for
  // them inside it: its own vmcnt count ignores the direct loads issued there, so a wait it
  // placed before the first use of kf/vf would also wait for the next tile's loads.
  wait_loads();
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(kf[kk]), "+v"(vf[kk]));
  if constexpr (DBIAS && CAUSAL) zero_dbias(0, min(t0 * kRows, Nq));  // tiles not visited
  int t = t0;
  for (; t < tm; ++t) {
    body(t, std::true_type{});
    pin(dk, dv);
  }
  for (; t < t1; ++t) {
    body(t, std::false_type{});
    pin(dk, dv);
  }

  // dK^T and dV^T: lane column = key, element i = dim 32db + 8(i/4) + 4g + i%4. They go out
  // through LDS in whole row segments (store_rows_staged), once every wave has finished
  // with the Q/dO stages.
  wait_loads();
  wg_barrier();
  static_assert((kT / 64) * 32 * 64 * 4 <= (int)sizeof(smem), "epilogue staging exceeds the LDS");
  char* const stg = smem + w * (32 * 64 * 4);
  float* const kout = p.dk + pv.kbase + (size_t)kw0 * rs;
  float* const vout = p.dv + pv.kbase + (size_t)kw0 * rs;
  store_rows_staged<D>(dk, p.scale, stg, kout, (size_t)rs, Nk - kw0, lane);
  store_rows_staged<D>(dv, 1.f, stg, vout, (size_t)rs, Nk - kw0, lane);
}

// ---------------------------------------------------------------- dQ

// BIAS: the scores carry the additive bias of fa_fwd_bias. Each wave stages the bias of its
// own 32 query rows for the current 64-key tile (4 KB, one buffer per wave) with direct
// loads issued right after the tile's barrier, and reads 4 keys per 8-byte read in the
// S^T layout (one query per lane column); 16-byte chunks are XOR-swizzled by (row / 2) % 8
// against bank conflicts (as in the biased prefill).
template <int D, bool CAUSAL, bool BIAS = false, bool VARLEN = false>
__global__ __launch_bounds__(kT, 2) void bwd_dq_kernel(BwdParams p) {
  using C = BCfg<D>;
  constexpr int STAGE = 2 * C::TILEB;  // K tile, V tile
  constexpr int WBIAS = 32 * kRows * 2;                   // one wave's bias rows of a tile
  constexpr int BOFF = 2 * STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + (BIAS ? 4 * WBIAS : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int col = lane & 31;

  int bh, qt;
  // (not compiled into the biased instances: it costs them registers)
  if (VARLEN || BIAS || p.tail_q.draws == 0) {
    map_block(blockIdx.x, gridDim.x, p.nqt, p.hpg_q, CAUSAL, bh, qt);
  } else {
    __shared__ int s_item;
    if (!map_block_tail(p.tail_q, &g_tail_tickets[p.slot_q], &s_item, p.nqt, p.hpg_q, CAUSAL, bh, qt))
      return;  // the pool was empty: no item for this workgroup
  }
  const int q0 = qt * kBwdQueryRows;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + col;
  static_assert(!(BIAS && VARLEN), "the bias is offered for dense batches only");
  const PairView pv = pair_view<D, VARLEN>(p, bh);
  const int Nq = pv.Nq, Nk = pv.Nk, off = pv.off, rs = pv.rs;
  if (VARLEN && q0 >= Nq) return;  // the whole workgroup: this sequence has no such rows

  const __bf16* __restrict__ qh = (const __bf16*)p.q + pv.qbase;
  const __bf16* __restrict__ doh = (const __bf16*)p.dout + pv.qbase;
  const __bf16* __restrict__ kh = (const __bf16*)p.k + pv.kbase;
  const __bf16* __restrict__ vh = (const __bf16*)p.v + pv.kbase;
  const float* __restrict__ wsh = p.ws + (size_t)bh * p.Nq_pad * 2;

  // Q and dO rows of this lane's query: B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (qrow < Nq) {
      qf[kk] = *(const bf16x8*)(qh + (size_t)qrow * rs + 16 * kk + 8 * g);
      df[kk] = *(const bf16x8*)(doh + (size_t)qrow * rs + 16 * kk + 8 * g);
    } else {
      qf[kk] = bf16x8{};
      df[kk] = bf16x8{};
    }
  }
  // padding rows (qrow >= Nq, < Nq_pad) carry LSE2 = +inf: their probabilities are 0
  float lse2 = wsh[stat_index(qrow)];
  float dsum = wsh[stat_index(qrow) + 64];
  // Pass the row data through an empty asm before the first tile load: the compiler then
  // waits for these loads once, here, instead of waiting inside the loop with a count
  // that ignores the in-flight tile loads (which would hold each step until the next
  // tile had landed).
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qf[kk]), "+v"(df[kk]));
  asm volatile("" : "+v"(lse2), "+v"(dsum));

  int kv_end = Nk;
  int wave_kv_end = (wq0 < Nq) ? Nk : 0;
  if (CAUSAL) {
    const int last_q = min(q0 + kBwdQueryRows, Nq) - 1;
    kv_end = min(Nk, last_q + off + 1);
    if (wq0 < Nq) wave_kv_end = min(Nk, min(wq0 + 31, Nq - 1) + off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + kRows - 1) / kRows : 0;

  const int lrow = tid / C::CHR;
  const uint32_t lchunk = 16u * (uint32_t)((tid % C::CHR) ^ bswz<C::CHR>(lrow));
  auto stage = [&](int i) -> char* { return smem + i * STAGE; };
  auto issue = [&](int t, char* st) {
    const int r0 = t * kRows;
#pragma unroll
    for (int n = 0; n < C::LOADS; ++n) {
      const int row = min(lrow + n * C::ROWSTEP, Nk - 1 - r0);  // rows past Nk repeat row Nk-1
      const uint32_t loff = (uint32_t)(row * rs * 2) + lchunk;
      const uint32_t dst = (uint32_t)((n * kT + 64 * w) * 16);
      dma16(kh + (size_t)r0 * rs, loff, lds_addr(st + dst));
      dma16(vh + (size_t)r0 * rs, loff, lds_addr(st + C::TILEB + dst));
    }
  };

  // Bias rows of this wave (BIAS only): row r of the wave (query wq0 + r, clamped to Nq-1)
  // starts at bwv + r*bsq; direct load n of lane L fills row 8n + L/8, chunk position L%8,
  // which holds chunk position ^ ((row / 2) % 8) of the row's 64 keys.
  const uint16_t* bwv = nullptr;
  char* const bwl = smem + BOFF + w * WBIAS;
  uint32_t boff[4];
  if constexpr (BIAS) {
    const int b = bh / p.H;
    const int r0 = min(wq0, Nq - 1);
    bwv = (const uint16_t*)p.bias + (size_t)b * p.bsb + (size_t)(bh - b * p.H) * p.bsh + (size_t)r0 * p.bsq;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int r = 8 * n + (lane >> 3);
      const int dr = min(wq0 + r, Nq - 1) - r0;
      boff[n] = (uint32_t)((long long)dr * p.bsq * 2) + 16u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    }
  }
  auto bias_issue = [&](int t) {
    const int ka = t * kRows;
    const char* base = (const char*)(bwv + ka);
    if (ka + kRows <= Nk) {
#pragma unroll
      for (int n = 0; n < 4; ++n) dma16(base, boff[n], lds_addr(bwl + n * 64 * 16));
      return;
    }
    // the key tail: chunks at or past Nk take the chunk of key Nk-1 (masked anyway)
    const int cmax = (Nk - 1 - ka) >> 3;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int r = 8 * n + (lane >> 3);
      const int dr = min(wq0 + r, Nq - 1) - min(wq0, Nq - 1);
      const int ch = min((lane & 7) ^ ((r >> 1) & 7), cmax);
      const uint32_t off = (uint32_t)((long long)dr * p.bsq * 2) + 16u * (uint32_t)ch;
      dma16(base, off, lds_addr(bwl + n * 64 * 16));
    }
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};

  if (ntiles > 0) issue(0, stage(0));
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    wait_loads();
    wg_barrier();
    // this wave's bias rows of tile t, before the next tile's loads (loads complete in order)
    if constexpr (BIAS) bias_issue(t);
    if (t + 1 < ntiles) issue(t + 1, stage(cur ^ 1));
    const char* Ks = stage(cur);
    const char* Vs = Ks + C::TILEB;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ka = t * kRows + 32 * kb;  // first key of this 32-key block
      if (ka >= wave_kv_end) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma(rfrag<D>(Ks, 32 * kb + col, 2 * kk + g), qf[kk], s);
        dp = mfma(rfrag<D>(Vs, 32 * kb + col, 2 * kk + g), df[kk], dp);
      }
      // element i: key ka + 8(i/4) + 4g + i%4, query qrow
      const bool need_mask = (ka + 32 > Nk) || (CAUSAL && ka + 31 > wq0 + off);
      const int lim = (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - ka - 4 * g;
      if constexpr (BIAS) {
        // s <- s * scale + bias, in natural-log units; keys ka + 8q + 4g + 0..3 sit at byte
        // 8g of chunk position (4kb + q) ^ ((col / 2) % 8) of this lane's row
        if (kb == 0) {
          if (t + 1 < ntiles)
            wait_loads_but<2 * C::LOADS>();  // the bias, not the next tile's K and V
          else
            wait_loads();
        }
        const char* brow = bwl + col * (kRows * 2);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const v4i16 raw = *(const v4i16*)(brow + (((4 * kb + qd) ^ ((col >> 1) & 7)) << 4) + 8 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[4 * qd + e] = __builtin_fmaf(s[4 * qd + e], p.scale,
                                           __uint_as_float((uint32_t)(uint16_t)raw[e] << 16));
        }
      }
      // P and dS; the mask in a branch of its own (it is needed only on the diagonal and the
      // key tail), so the other blocks carry no compare and select per element (-5% dQ time)
      bf16x8 dsb[2];
      const float cexp = BIAS ? kLog2e : p.c;
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cexp, -lse2));
          if (8 * (i >> 2) + (i & 3) > lim) pe = 0.f;
          dsb[i >> 3][i & 7] = (__bf16)(pe * (dp[i] - dsum));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cexp, -lse2));
          dsb[i >> 3][i & 7] = (__bf16)(pe * (dp[i] - dsum));
        }
      }
#pragma unroll
      for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dq[db] = mfma(tfrag<D>(Ks, 32 * kb + 16 * st2, db, lane), dsb[st2], dq[db]);
    }
  }

  // dQ^T: lane column = query, element i = dim 32db + 8(i/4) + 4g + i%4. It goes out through
  // LDS in whole row segments (store_rows_staged), once every wave has finished with the
  // K/V stages.
  wait_loads();
  wg_barrier();
  static_assert((kT / 64) * 32 * 64 * 4 <= (int)sizeof(smem), "epilogue staging exceeds the LDS");
  store_rows_staged<D>(dq, p.scale, smem + w * (32 * 64 * 4), p.dq + pv.qbase + (size_t)wq0 * rs, (size_t)rs,
                       Nq - wq0, lane);
}

template <int D, bool BIAS = false>
hipError_t launch(const BwdParams& prm, bool causal, hipStream_t s) {
  BwdParams p = prm;
  constexpr int RPB = 256 / (D / 8);
  const long long rows = (long long)p.BH * p.Nq_pad;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nkv = (unsigned)(p.tail_kv.draws ? 8 * p.tail_kv.s + p.tail_kv.draws : p.BH * p.nkt);
  const unsigned nq = (unsigned)(p.tail_q.draws ? 8 * p.tail_q.s + p.tail_q.draws : p.BH * p.nqt);
  if constexpr (BIAS) {
    if (causal) {
      if (p.dbias)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true, true>), dim3(nkv), dim3(kT), 0, s, p);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true, false>), dim3(nkv), dim3(kT), 0, s, p);
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, true>), dim3(nq), dim3(kT), 0, s, p);
    } else {
      if (p.dbias)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true, true>), dim3(nkv), dim3(kT), 0, s, p);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true, false>), dim3(nkv), dim3(kT), 0, s, p);
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, true>), dim3(nq), dim3(kT), 0, s, p);
    }
  } else if (causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3(nkv), dim3(kT), 0, s, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3(nq), dim3(kT), 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3(nkv), dim3(kT), 0, s, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3(nq), dim3(kT), 0, s, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_varlen(const BwdParams& prm, bool causal, hipStream_t s) {
  BwdParams p = prm;
  constexpr int RPB = 256 / (D / 8);
  const long long rows = (long long)p.BH * p.Nq_pad;
  hipLaunchKernelGGL((bwd_pre_kernel<D, true>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned nkv = (unsigned)(p.BH * p.nkt), nq = (unsigned)(p.BH * p.nqt);
  if (causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false, false, true>), dim3(nkv), dim3(kT), 0, s, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, true>), dim3(nq), dim3(kT), 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false, false, true>), dim3(nkv), dim3(kT), 0, s, p);
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, true>), dim3(nq), dim3(kT), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_varlen(const BwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch_varlen<128>(p, causal, s);
  return launch_varlen<64>(p, causal, s);
}

hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128>(p, causal, s);
  return launch<64>(p, causal, s);
}

hipError_t launch_bwd_bias(const BwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, true>(p, causal, s);
  return launch<64, true>(p, causal, s);
}

}  // namespace fa
