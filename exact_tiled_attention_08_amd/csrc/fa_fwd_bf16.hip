// Attention forward for bfloat16 Q/K/V on gfx950: bf16 MFMA, float32 accumulation.
//
// One workgroup owns BR = 256 query rows of one (b, h); each of its 8 waves owns 32 rows.
// K and V stream through LDS in tiles of BC keys, and each wave folds every tile into its
// running state with the online-softmax recurrence: "FlashAttention: Attention Is Limited
// by Memory, Not Math", section "How tiling and online softmax stay exact" (running max m
// and sum l; previous sums rescaled by exp(m_old - m_new) when the max rises; divide by l
// once at the end), and "Explain FlashAttention ...", section "Keep only the state needed
// for the final weighted average". Each query block is read once and every key/value block
// streams past it ("Flash Attention Optimization", section "Active recall", question 6
// and its answer); the query tiles of all heads are independent workgroups
// ("FlashAttention 1, 2 and 3": parallel over sequence length as well as batch and heads).
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
// Schedule: the 8 waves form two groups of 4 (one wave of each group per SIMD). A group
// alternates a matrix phase (S for the next tile and PV for the current tile, all MFMA)
// with a vector phase (mask, online softmax, rescale of O), and the groups run half a
// step apart, separated by workgroup barriers: while one group's waves keep a SIMD's
// matrix core busy, the other group's waves use its vector ALU. Group 0 issues the direct
// loads of K tiles and group 1 those of V tiles, each two phases ahead of the first use.
//
// Packed variable-length batches (VARLEN): the same kernel over [total][H][d] tensors with
// per-sequence row offsets; a workgroup finds its sequence's rows and lengths, exits at
// once when its query tile lies past the sequence's end, and otherwise runs unchanged with
// a row stride of H*d elements (masks use positions inside the sequence). Its (b, h) pairs
// are numbered head-major so that every XCD gets a share of every sequence.
//
// Additive bias (BIAS): the bias is added to the scaled scores before the softmax
// ("Explain FlashAttention ...", section "Keep only the state needed for the final
// weighted average": scaled scores plus the intended mask or bias). Each wave streams the
// bias of its own 32 query rows for a tile (32 x 64 bfloat16, 4 KB) from global memory
// straight into its own double-buffered LDS area, issuing tile j+2 while it folds in tile
// j+1, and waits for exactly the loads it needs (loads complete in issue order), so the
// K/V stream is never held up behind the bias. Rows are stored with the 16-byte chunk
// index XORed with (row / 2) % 8, which leaves at most two lanes of a half-wave on one
// bank pair when each lane reads its row's 4 keys. The score becomes s * scale + bias
// (one fma after widening the bias) and the softmax takes it to log2 units with its own
// fma, so the bias costs two vector ops per score; masked keys stay -inf whatever their
// bias.
//
// Rescaling: the offset is always the exact running max, so the largest weight of a row
// is exactly 1 and survives the rounding of P to bfloat16 without error (an offset that
// lags the max would leave the dominant weight at 2^delta, rounded by up to 2^-9 of its
// size); the multiply of O is skipped when no row of the wave raised its max.
#include <utility>

#include "fa_internal.h"

namespace fa {
namespace {

// Ticket counters of the dynamic tail (map_block_tail), zero at load and put back to zero
// by the last ticket of every launch.
__device__ unsigned g_tail_tickets[kTailSlots];

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kNW = 8;  // waves per workgroup: two groups of four

// Race check (a separate build, libfa_ldscheck.so, defines FA_LDS_POISON=1; the product
// library does not): right before a direct load is issued into an LDS slot, the issuing
// lane first overwrites that slot with NaN and waits for the write. The slot's previous
// tile has then had its last reader (the barriers are meant to guarantee it), and the new
// tile has not landed yet, so a wave that reads a slot too late (stale tile) or too early
// (not yet landed) reads NaN, which turns into NaN or wrong values in O: with no race the
// results are bitwise those of the product library.
#ifndef FA_LDS_POISON
#define FA_LDS_POISON 0
#endif
constexpr bool kPoison = FA_LDS_POISON != 0;

// Fills one 16-byte LDS slot with NaN bit patterns (every bfloat16 half is 0xFFFF) and waits
// until the write has completed, so that a direct load issued next lands on top of it.
__device__ __forceinline__ void poison16(char* lds_slot) {
  *(uint4*)lds_slot = make_uint4(0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// dma16 with the non-temporal hint, for data read exactly once (the bias): it then does not
// push out of L2 the K/V tiles that the other query tiles of a head read again (measured:
// 5% faster biased prefill, no change in results). M0 is declared clobbered as in dma16.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_once(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory", "m0");
}
#pragma clang diagnostic pop

template <int D, int BC>
struct Cfg {
  static constexpr int BR = 32 * kNW;         // query rows per workgroup
  static constexpr int T = 64 * kNW;          // threads per workgroup
  static constexpr int TL = T / 2;            // threads that load one tensor (one group)
  static constexpr int ROWB = D * 2;          // bytes per K or V row in LDS (unpadded)
  static constexpr int CHR = D / 8;           // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;     // bytes of one K (or V) tile
  static constexpr int LDS = 4 * TILEB;       // two K buffers, two V buffers
  static constexpr int SLOTS = BC * CHR;      // 16-byte slots per tile
  static constexpr int LOADS = SLOTS / TL;    // direct loads per thread per tile
  static constexpr int ROWSTEP = TL / CHR;    // rows between a thread's successive slots
  static_assert(D % 32 == 0 && BC % 32 == 0 && CHR >= 8, "tile shape");
  static_assert(SLOTS % TL == 0 && TL % CHR == 0, "slots must split evenly over threads");
  static_assert(ROWSTEP % 16 == 0, "swizzles must repeat every ROWSTEP rows");
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

// Bias staging of the BIAS kernel: per wave and buffer, 32 rows x BC keys of bfloat16.
template <int BC>
struct BiasCfg {
  static constexpr int ROWB = BC * 2;           // bytes per row
  static constexpr int WAVEB = 32 * ROWB;       // bytes per wave and buffer
  static constexpr int LDS = 2 * kNW * WAVEB;   // two buffers for every wave
  static constexpr int LOADS = WAVEB / (64 * 16);  // direct loads per lane per tile
  static_assert(BC == 64, "the bias swizzle assumes 8 chunks of 16 bytes per row");
};

template <int D, int BC, bool CAUSAL, bool VARLEN, bool BIAS>
__global__ __launch_bounds__(64 * kNW, 2) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, BC>;
  static_assert(!(BIAS && VARLEN), "bias is offered for dense batches only");
  using BCfg = BiasCfg<BIAS ? BC : 64>;
  constexpr int BIASLDS = BIAS ? BCfg::LDS : 0;
  // Q staging (no bias): each wave's 32 query rows, loaded global -> LDS in whole rows
  constexpr int QSTAGE = BIAS ? 0 : kNW * 32 * D * 2;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS + BIASLDS + QSTAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
  const bool loader = w < kNW / 2;                          // group 0 issues the loads
  const int g = lane >> 5;
  const int col = lane & 31;

  int bh, qt;
  // (the biased kernel, bound by HBM, measured no gain from the dynamic tail and keeps the
  // fixed map)
  if (VARLEN || BIAS || p.tail.draws == 0) {
    map_block(blockIdx.x, gridDim.x, p.nqt, p.hpg, CAUSAL, bh, qt);
  } else {
    // the draw's result passes through K buffer 1, which no load writes before the first
    // barrier of the prologue (every wave has read it by then)
    int* const s_item = (int*)(smem + C::TILEB);
    if (!map_block_tail(p.tail, &g_tail_tickets[p.tail_slot], s_item, p.nqt, p.hpg, CAUSAL, bh, qt))
      return;  // the pool was empty: no item for this workgroup
  }
  const int q0 = qt * C::BR;
  const int wq0 = q0 + 32 * w;  // first query row of this wave
  const int qrow = wq0 + col;   // this lane's query row

  // Rows of this (b, h): Nq queries and Nk keys, `rs` elements apart (a dense [B][H][N][d]
  // tensor: d; a packed [total][H][d] batch: H*d). Causal offset: key position of query 0.
  int Nq = p.Nq, Nk = p.Nk, off = p.off;
  const uint16_t* __restrict__ qh;
  const uint16_t* __restrict__ kh;
  const uint16_t* __restrict__ vh;
  float* __restrict__ oh;
  float* __restrict__ lh;
  if (VARLEN) {
    // pairs are numbered head-major (h * B + b): the contiguous run of pairs that the block
    // map gives one XCD then spans every sequence for a few heads, so the XCDs get equal
    // work however unequal the sequences are, and a head's K/V still stays in one L2
    const int h = bh / p.B;
    const int b = bh - h * p.B;
    // offsets clamped into the packed tensors, so malformed ones cannot read outside them
    const int qs = min(max(p.cu_q[b], 0), p.total_q);
    const int ks = min(max(p.cu_k[b], 0), p.total_k);
    Nq = min(max(p.cu_q[b + 1], qs), p.total_q) - qs;
    Nk = min(max(p.cu_k[b + 1], ks), p.total_k) - ks;
    off = p.top_left ? 0 : Nk - Nq;
    if (q0 >= Nq) return;  // the whole workgroup: this sequence has no rows in this tile
    qh = (const uint16_t*)p.q + ((size_t)qs * p.H + h) * D;
    kh = (const uint16_t*)p.k + ((size_t)ks * p.H + h) * D;
    vh = (const uint16_t*)p.v + ((size_t)ks * p.H + h) * D;
    oh = p.o + ((size_t)qs * p.H + h) * D;
    lh = p.lse ? p.lse + (size_t)h * p.total_q + qs : nullptr;
  } else {
    qh = (const uint16_t*)p.q + (size_t)bh * Nq * D;
    kh = (const uint16_t*)p.k + (size_t)bh * Nk * D;
    vh = (const uint16_t*)p.v + (size_t)bh * Nk * D;
    oh = p.o + (size_t)bh * Nq * D;
    lh = p.lse ? p.lse + (size_t)bh * Nq : nullptr;
  }
  const int rs = VARLEN ? p.H * D : D;  // elements between consecutive rows

  // Bias rows of this wave: element (row wq0 + r, key j) at bw + dr*bsq + j, where the
  // row is clamped to Nq-1 (rows past Nq are computed but never stored) and dr = the
  // clamped row minus bias_r0.
  const uint16_t* bw = nullptr;
  const int bias_r0 = min(wq0, Nq - 1);
  if constexpr (BIAS) {
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    bw = (const uint16_t*)p.bias + (size_t)b * p.bsb + (size_t)h * p.bsh + (size_t)bias_r0 * p.bsq;
  }

  // Q tile stays in VGPRs for the whole key loop, as the B operand of S^T = K Q^T. A lane
  // needs 16-byte pieces of one row, so loading them directly reads 32 bytes of each of 32
  // rows per instruction. Without a bias, the wave's rows instead go global -> LDS in whole
  // rows (direct loads, chunk c of row r at chunk position c ^ (r % CHR), issued together
  // with the first K/V tile) and are read into VGPRs once those loads have landed (same
  // process, bitwise-identical results: +0.35-0.5% on the three bf16 prefill shapes; a
  // timing-only copy that loaded the same bytes contiguously straight into the wrong lanes
  // gained 1.5% at N = 8192, so the LDS round trip costs most of what the pattern saves).
  // Rows past Nq load row Nq - 1: their scores stay finite, and they are never stored.
  bf16x8 qb[D / 16];
  char* const qstage = smem + C::LDS + BIASLDS + w * (32 * D * 2);
  if constexpr (BIAS) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      if (qrow < Nq)
        qb[kk] = *(const bf16x8*)(qh + (size_t)qrow * rs + 16 * kk + 8 * g);
      else
        qb[kk] = bf16x8{};
    }
  } else {
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    const uint32_t qlds = (uint32_t)(uintptr_t)((lds_char*)qstage);
    const int qr0 = min(wq0, Nq - 1);        // base row (a wave past Nq re-reads row Nq - 1)
    const int rlast = min(31, Nq - 1 - qr0);  // last row from the base that lies below Nq
    const char* const qbase = (const char*)qh + (size_t)qr0 * rs * 2;
    // an opaque copy of the lane index: the epilogue's store addresses have the same form,
    // and the compiler would otherwise keep these terms alive across the key loop (spills)
    int ql = lane;
    asm volatile("" : "+v"(ql));
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const int slot = 64 * n + ql;
      const int r = slot / CPR, pos = slot % CPR;
      const int c = pos ^ (r % CPR);
      dma16(qbase, (uint32_t)(min(r, rlast) * rs * 2 + 16 * c), qlds + 1024u * n);
    }
  }

  // Key tiles this workgroup visits, and the key bound of this wave (causal).
  int kv_end = Nk;
  int wave_kv_end = (wq0 < Nq) ? Nk : 0;
  if (CAUSAL) {
    const int last_q = min(q0 + C::BR, Nq) - 1;
    kv_end = min(Nk, last_q + off + 1);
    if (wq0 < Nq) wave_kv_end = min(Nk, min(wq0 + 31, Nq - 1) + off + 1);
  }
  const int ntiles = kv_end > 0 ? (kv_end + BC - 1) / BC : 0;

  // Direct-load slots of a loading thread: slot s = n*TL + tid -> row s / CHR, chunk
  // position s % CHR; the chunk fetched is the one the swizzle stores at that position.
  // Both swizzles depend only on row bits that repeat every ROWSTEP rows, so one byte
  // offset per tensor serves all of the thread's slots.
  const int lrow = (tid % C::TL) / C::CHR;
  const int lpos = tid % C::CHR;
  const uint32_t koff = (uint32_t)(lrow * C::ROWB + 16 * swz_k<C::CHR>(lrow, lpos));
  const uint32_t voff = (uint32_t)(lrow * C::ROWB + 16 * swz_v<C::CHR>(lrow, lpos));
  auto kbuf = [&](int i) -> char* { return smem + i * C::TILEB; };
  auto vbuf = [&](int i) -> char* { return smem + (2 + i) * C::TILEB; };
  // Group 0 loads the K tiles and group 1 the V tiles. One direct load (slot group n of
  // tile t) of this wave into LDS buffer dst: key rows past Nk re-read row Nk-1, so the
  // per-lane offset is the clamped row's (< 2^31 bytes: Nk * d <= 2^30) plus the lane's
  // swizzled chunk within the row, against the tile's 64-bit base.
  const uint16_t* const lbase = loader ? kh : vh;
  const uint32_t lchunk = (loader ? koff : voff) - (uint32_t)(lrow * C::ROWB);
  const int wg4 = w & 3;  // wave index within its group
  // Where group 1 issues its V tiles. Issuing one tile's direct loads holds the issuing
  // waves for ~300-500 cycles (the CU accepts them at ~50-90 B/clk), so the issue belongs
  // where a group has time to spare. At d = 128 (no bias) group 1 loads V_{j+1} at the start
  // of its matrix phase of step j, into the buffer of V_{j-1}, which both groups finished
  // reading at the barrier before; the vector phase it used to end, and which the other
  // group's matrix phase waited for, then carries no load. Measured in one process: +1.2 to
  // +1.5% at N = 8192 and +0.5 to +1.1% at N = 30000, bitwise-identical results; at d = 64
  // it measured -0.9%, so there (and in the bias kernel, whose loads interleave with its
  // bias tiles) group 1 keeps loading V_{j+2} at the end of its vector phase.
  constexpr bool kVEarly = !BIAS && D == 128;
  auto dma = [&](int t, char* dst, int n) {
    const int kv0 = t * BC;
    if constexpr (kPoison) poison16(dst + (n * C::TL + 64 * wg4 + lane) * 16);
    const uint32_t lds = (uint32_t)(uintptr_t)((lds_char*)(dst + (n * C::TL + 64 * wg4) * 16));
    const int row = min(lrow + n * C::ROWSTEP, Nk - 1 - kv0);
    dma16((const char*)lbase + (size_t)kv0 * rs * 2, (uint32_t)(row * rs * 2) + lchunk, lds);
  };
  // Whole tiles (every row below Nk) need no clamp: the lane's offset from its row-group
  // base is then the same for every slot and tile (one loop-invariant VGPR) and the row
  // step goes into the scalar base, so issuing a load costs no vector instruction.
  const uint32_t loff = (uint32_t)(lrow * rs * 2) + lchunk;
  auto issue = [&](int t, char* dst) {
    const int kv0 = t * BC;
    if (kv0 + BC <= Nk) {
      if constexpr (kPoison)
        for (int n = 0; n < C::LOADS; ++n) poison16(dst + (n * C::TL + 64 * wg4 + lane) * 16);
      const uint32_t lds0 = (uint32_t)(uintptr_t)((lds_char*)(dst + 64 * wg4 * 16));
      [&]<int... N>(std::integer_sequence<int, N...>) {
        (dma16_at<N * C::TL * 16>((const char*)lbase + (size_t)(kv0 + N * C::ROWSTEP) * rs * 2, loff, lds0), ...);
      }(std::make_integer_sequence<int, C::LOADS>{});
    } else {
#pragma unroll
      for (int n = 0; n < C::LOADS; ++n) dma(t, dst, n);  // the key tail: rows clamped
    }
  };
  // Bias of key tile t into this wave's buffer t % 2. Direct load n of lane L fills LDS
  // slot 64n + L: row 8n + L/8, chunk position L%8, which holds the row's chunk
  // position ^ ((row / 2) % 8). A chunk that starts at or past Nk is replaced by the
  // chunk holding key Nk-1 (its keys are masked anyway), so the reads stay inside each
  // row's first Nk elements rounded up to a multiple of 8.
  char* const bias_lds = smem + C::LDS;
  auto bias_buf = [&](int t) { return bias_lds + ((t & 1) * kNW + w) * BCfg::WAVEB; };
  // Lane offsets of whole tiles (no chunk starts at or past Nk) do not depend on the
  // tile: computed once.
  uint32_t boff[BCfg::LOADS];
  if constexpr (BIAS) {
#pragma unroll
    for (int n = 0; n < BCfg::LOADS; ++n) {
      const int dr = min(wq0 + 8 * n + (lane >> 3), Nq - 1) - bias_r0;
      const int ch = (lane & 7) ^ (((n & 1) << 2) | (lane >> 4));
      boff[n] = (uint32_t)((long long)dr * p.bsq * 2) + 16u * (uint32_t)ch;
    }
  }
  auto bias_issue = [&](int t) {
    const int kv0 = t * BC;
    const int cmax = (Nk - 1 - kv0) >> 3;
    const char* base = (const char*)(bw + kv0);
    char* dst = bias_buf(t);
    if constexpr (kPoison)
      for (int n = 0; n < BCfg::LOADS; ++n) poison16(dst + (n * 64 + lane) * 16);
    if (kv0 + BC <= Nk) {
#pragma unroll
      for (int n = 0; n < BCfg::LOADS; ++n)
        dma16_once(base, boff[n], (uint32_t)(uintptr_t)((lds_char*)(dst + n * 64 * 16)));
      return;
    }
#pragma unroll
    for (int n = 0; n < BCfg::LOADS; ++n) {
      const int row = 8 * n + (lane >> 3);
      const int dr = min(wq0 + row, Nq - 1) - bias_r0;
      const int ch = min((lane & 7) ^ (((n & 1) << 2) | (lane >> 4)), cmax);
      const uint32_t lds = (uint32_t)(uintptr_t)((lds_char*)(dst + n * 64 * 16));
      dma16_once(base, (uint32_t)((long long)dr * p.bsq * 2) + 16u * (uint32_t)ch, lds);
    }
  };
  // s <- s * scale + bias for tile t (this lane's query row, its 16 keys per 32-key
  // block: 32kb + 8(i/4) + 4g + i%4, one 8-byte read per 4 keys).
  auto add_bias = [&](int t, f32x16 (&s)[BC / 32]) {
    const char* row = bias_buf(t) + col * BCfg::ROWB;
    const int sw = (col >> 1) & 7;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const v4i16 raw = *(const v4i16*)(row + (((4 * kb + qd) ^ sw) << 4) + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float bv = __uint_as_float((uint32_t)(uint16_t)raw[e] << 16);
          s[kb][4 * qd + e] = __builtin_fmaf(s[kb][4 * qd + e], p.scale, bv);
        }
      }
  };

  // K fragment (A operand of S^T = K_j Q_i^T, BC keys x 32 queries per wave) of key block
  // kb and 16-dim contraction step kk.
  auto kfrag = [&](const char* Ks, int kb, int kk) {
    const int r = 32 * kb + col;
    return *(const bf16x8*)(Ks + r * C::ROWB + swz_k<C::CHR>(r, 2 * kk + g) * 16);
  };
  // Mask on absolute positions, only for tiles that cross the key tail or the diagonal
  // (a tile past the wave's keys is masked out entirely):
  // key kv0 + 32kb + 8(i/4) + 4g + i%4 is visible iff its in-tile offset <= lim.
  auto needs_mask = [&](int t) {
    const int kv0 = t * BC;
    return (kv0 + BC > Nk) || (CAUSAL && kv0 + BC - 1 > wq0 + off) || (kv0 >= wave_kv_end);
  };
  auto mask_s = [&](int t, f32x16 (&s)[BC / 32]) {
    const int lim = (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - t * BC - 4 * g;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kb + 8 * (i >> 2) + (i & 3) > lim) s[kb][i] = -INFINITY;
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY;  // running max of this lane's row, in log2 units (score * c)
  float l = 0.f;        // running sum over this lane's half of the keys

  // Online softmax of one tile; O is rescaled here, after the previous tile's PV and
  // before this tile's, and only when some row of the wave raised its max. With a bias
  // the scores arrive already scaled (natural-log units).
  const float cs = BIAS ? kLog2e : p.c;
  auto softmax = [&](f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 16]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    const float mt = wave_half_max(mx) * cs;  // tile row max, log2 units (-inf if masked)
    const bool raise = mt > m;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m - mt) : 1.f;  // 0 when m was -inf
    m = raise ? mt : m;
    const float m_use = (m == -INFINITY) ? 0.f : m;  // nothing visible yet: weights are 0
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], cs, -m_use));
        lsum += e;
        pb[2 * kb + (i >> 3)][i & 7] = (__bf16)e;  // round to nearest even
      }
    l = l * alpha + lsum;
    if (__any(raise)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
  };
  // O^T += V_j^T P^T; the V^T operand comes from two transpose reads per 16-key step.
  const int trG = (lane >> 4) & 1;  // which 16 of the 32 output dims
  const int trj = lane & 15;
  // The V^T fragment of (16-key step kc, 32-dim block db): two transpose reads.
  auto vfrag = [&](const char* Vs, int kc, int db) {
    bf16x4 half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * kc + 8 * h + 4 * g + (trj >> 2);
      const int cbyte = 64 * db + 32 * trG + 8 * (trj & 3);
      const int addr = r * C::ROWB + swz_v<C::CHR>(r, cbyte >> 4) * 16 + (cbyte & 15);
      half[h] = __builtin_bit_cast(
          bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(Vs + addr)));
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Matrix phase: O^T += V_j^T P_j^T (MFMAs 0 .. NPV-1), then S^T = K_{j+1} Q^T (MFMAs
  // NPV .. NF-1, into freshly zeroed accumulators). In each product the accumulators
  // advance together along the contraction, so consecutive MFMAs are independent; the A
  // fragment of MFMA f is read from LDS RING-1 MFMAs ahead, across the boundary between
  // the two products.
  constexpr int NDB = D / 32, NKB = BC / 32;
  constexpr int NPV = NDB * (BC / 16), NF = NPV + NKB * (D / 16), RING = 4;
  auto afrag = [&](const char* Vs, const char* Ks, int f) {
    return f < NPV ? vfrag(Vs, f / NDB, f % NDB) : kfrag(Ks, (f - NPV) % NKB, (f - NPV) / NKB);
  };
  // With WITH_S false (the last tile) only the PV MFMAs run.
  auto matrix = [&]<bool WITH_S>(const char* Vs, const char* Ks, const bf16x8 (&pb)[BC / 16],
                                 f32x16 (&s)[BC / 32]) {
    constexpr int NM = WITH_S ? NF : NPV;
    bf16x8 fr[RING];
#pragma unroll
    for (int f = 0; f < RING - 1; ++f) fr[f] = afrag(Vs, Ks, f);
#pragma unroll
    for (int f = 0; f < NM; ++f) {
      const int fn = f + RING - 1;
      if (fn < NM) fr[fn % RING] = afrag(Vs, Ks, fn);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this MFMA
      if (f < NPV) {
        oacc[f % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[f % RING], pb[f / NDB], oacc[f % NDB], 0, 0, 0);
      } else {
        const int g2 = f - NPV;
        s[g2 % NKB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fr[f % RING], qb[g2 / NKB], g2 < NKB ? f32x16{} : s[g2 % NKB], 0, 0, 0);
      }
    }
  };
  // Prologue only: S^T of tile 0.
  auto compute_s = [&](const char* Ks, f32x16 (&s)[BC / 32]) {
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(Ks, kb, kk), qb[kk], kk == 0 ? f32x16{} : s[kb], 0, 0, 0);
  };

  // Prologue: tile 0 lands in K and V buffer 0 (group 0 loads K, group 1 loads V); every
  // wave computes S and the softmax of tile 0; each group starts loading its tile 1.
  bf16x8 pb[BC / 16];
  f32x16 s[BC / 32];
  if (ntiles > 0) issue(0, loader ? kbuf(0) : vbuf(0));
  if constexpr (BIAS)
    if (ntiles > 0) bias_issue(0);
  // Q and tile 0 have landed. Waiting on every path with the builtin lets the compiler see
  // that the Q loads are complete, so it does not re-wait for them inside the loop (where
  // the wait would also stall on the in-flight tile loads that share the counter).
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unchanged
  if constexpr (!BIAS) {
    asm volatile("" ::: "memory");  // the Q rows are in LDS now
    constexpr int CPR = D / 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qb[kk] = *(const bf16x8*)(qstage + col * (D * 2) + (((2 * kk + g) ^ (col % CPR)) << 4));
  }
  // The compiler merges control flow so that some path into the loop bypasses that wait;
  // it would then wait for the Q loads again before the first S^T MFMA of every matrix
  // phase, and that vmcnt(0) would also stall on the tile loads just issued. Passing Q
  // through an empty asm makes the loop's Q registers values that no load is pending on.
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) asm volatile("" : "+v"(qb[kk]));
  if (ntiles > 0) {
    wg_barrier();
    if (ntiles > 1 && (loader || !kVEarly)) issue(1, loader ? kbuf(1) : vbuf(1));
    if constexpr (BIAS)
      if (ntiles > 1) bias_issue(1);
    if (wave_kv_end > 0) {
      compute_s(kbuf(0), s);
      if constexpr (BIAS) add_bias(0, s);
      if (needs_mask(0)) mask_s(0, s);
      softmax(s, pb);
    }
    if (!loader) wg_barrier();  // group 1 runs one phase behind group 0
  }

  // Step j < ntiles - 1: matrix phase (O += P_j V_j, then S for tile j+1 from K_{j+1}), a
  // barrier, then the vector phase (mask and softmax of tile j+1, rescale of O). Barriers
  // alternate between the groups' phases, so one group's matrix phase overlaps the other's
  // vector phase. Group 0 loads K_{j+2} at the start of its matrix phase of step j, into
  // the buffer of K_j, which both groups finished reading in their matrix phases of step
  // j-1. Group 1 loads V_{j+2} at the end of its vector phase of step j, into the buffer of
  // V_j (read by both groups' matrix phases of step j), or, with kVEarly, V_{j+1} at the
  // start of its matrix phase of step j, into the buffer of V_{j-1}. Each group waits for
  // its loads at the last barrier before their first reader: group 0 before its step j+1
  // matrix phase, group 1 before its mid-step barrier of step j+1 (of step j with
  // kVEarly: its V_{j+1} loads then have one matrix phase to land).
  //
  // With a bias, every wave also loads bias tile j+2 at the start of its vector phase of
  // step j, and reads bias tile j+1 (loaded one step earlier) in that phase. Group 0's
  // loads then run K_{j+1}, B_{j+1}, K_{j+2}, B_{j+2}, ...: at the start of step j it
  // waits for all but the last bias batch (that is, for K_{j+1}), and before reading
  // B_{j+1} for all but K_{j+2} and B_{j+2}. Group 1's wait for V_{j+1} also covers
  // B_{j+1}, issued before it.
  auto step = [&](int j, int cur) {  // cur = j & 1, passed as a constant by the unrolled loop
    if (loader) {  // K_{j+1}
      if constexpr (BIAS)
        wait_loads_but<BCfg::LOADS>();
      else
        wait_loads();
    }
    wg_barrier();
    if (loader && j + 2 < ntiles) issue(j + 2, kbuf(cur));
    if constexpr (kVEarly)
      if (!loader && j + 1 < ntiles) issue(j + 1, vbuf(cur ^ 1));  // V_{j+1}
    const bool active = j * BC < wave_kv_end;
    if (active) matrix.template operator()<true>(vbuf(cur), kbuf(cur ^ 1), pb, s);
    if (!loader) wait_loads();  // V_{j+1} (and the bias of tile j+1)
    wg_barrier();
    if constexpr (BIAS)
      if (j + 2 < ntiles) bias_issue(j + 2);
    if (active) {
      if constexpr (BIAS) {
        if (loader) {  // the bias of tile j+1
          if (j + 2 < ntiles)
            wait_loads_but<C::LOADS + BCfg::LOADS>();
          else
            wait_loads();
        }
        add_bias(j + 1, s);
      }
      if (needs_mask(j + 1)) mask_s(j + 1, s);
      softmax(s, pb);
    }
    if (!kVEarly && !loader && j + 2 < ntiles) issue(j + 2, vbuf(cur));  // V_{j+2}
  };
  // Step ntiles - 1: PV of the last tile only (there is no next tile to score). The
  // barriers keep the same count as a full step, so both groups end the loop together.
  auto last_step = [&](int j, int cur) {
    wg_barrier();
    if (j * BC < wave_kv_end) matrix.template operator()<false>(vbuf(cur), kbuf(cur ^ 1), pb, s);
    wg_barrier();
  };
  if (ntiles > 0) {
    // steps in pairs so that every LDS buffer address is a compile-time offset
    const int last = ntiles - 1;
    for (int j = 0; j < last; j += 2) {
      step(j, 0);
      if (j + 1 < last) step(j + 1, 1);
    }
    if (last & 1)
      last_step(last, 1);
    else
      last_step(last, 0);
    if (loader) wg_barrier();  // match group 1's extra barrier
    if constexpr (BIAS) wait_loads();  // a wave that skipped its last bias tile
  }

  // Epilogue: divide by l once; LSE = ln2 * (m + log2 l). Empty row: O = 0, LSE = -inf.
  // O leaves through this wave's own 8 KB of LDS, 64 columns at a time. A lane's registers
  // hold 16-byte pieces of one row, so storing them directly writes 32 bytes of each of 32
  // rows per instruction; read back row-major, each store writes whole 256-byte segments
  // of 4 rows (same process, bitwise-identical results: +1.1-1.2% at N = 8192, +1.4% on the
  // d = 64 shape). The stores are non-temporal: O is written once and never read here, and
  // streaming it past L2 leaves the K/V tiles there (a further +1.2% at N = 8192 and +1.6%
  // on the d = 64 shape; with the scattered 32-byte pattern the same hint had been slower).
  // Every wave has passed its last LDS read (the barrier after the last PV product), so the
  // K/V buffers are free. Chunk c of row r sits at chunk position c ^ (r % 16): both the
  // writes and the reads are then free of bank conflicts. (Group 0 staging in the K buffers
  // and storing while group 1 ran its last PV product measured slower.)
  const float lt = wave_half_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  constexpr int kStage = 32 * 64 * 4;  // one wave's area
  static_assert(kNW * kStage <= (int)sizeof(smem), "epilogue staging exceeds the LDS");
  char* const ot = smem + w * kStage;
#pragma unroll
  for (int hh = 0; hh < D / 64; ++hh) {
#pragma unroll
    for (int dbh = 0; dbh < 2; ++dbh)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int db = 2 * hh + dbh;
        f32x4 val;
        val[0] = oacc[db][4 * j + 0] * inv;
        val[1] = oacc[db][4 * j + 1] * inv;
        val[2] = oacc[db][4 * j + 2] * inv;
        val[3] = oacc[db][4 * j + 3] * inv;
        const int c = 8 * dbh + 2 * j + g;  // columns 64 hh + 4c .. 64 hh + 4c + 3
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
    float* const obase = oh + (size_t)(wq0 + (lane >> 4)) * rs + 64 * hh + 4 * c;
    if (wq0 + 32 <= Nq) {  // all 32 rows of the wave exist
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * rs));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (wq0 + 4 * i + (lane >> 4) < Nq)
          __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * rs));
    }
    asm volatile("" ::: "memory");
  }
  if (qrow < Nq && g == 0 && lh) lh[qrow] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

template <int D, int BC, bool VARLEN, bool BIAS = false>
hipError_t launch(const FwdParams& prm, bool causal, hipStream_t s) {
  FwdParams p = prm;
  const int total = p.tail.draws ? 8 * p.tail.s + p.tail.draws : p.BH * p.nqt;
  if (causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, true, VARLEN, BIAS>), dim3(total), dim3(64 * kNW), 0, s, p);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, false, VARLEN, BIAS>), dim3(total), dim3(64 * kNW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int fwd_bf16_block_rows(int) { return 32 * kNW; }

int fwd_bf16_key_tile(int d) { return d == 128 ? 96 : 128; }

hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, 96, false>(p, causal, s);
  return launch<64, 128, false>(p, causal, s);
}

hipError_t launch_fwd_bf16_varlen(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, 96, true>(p, causal, s);
  return launch<64, 128, true>(p, causal, s);
}

// 64-key tiles: they free the registers and LDS that the bias staging takes.
hipError_t launch_fwd_bf16_bias(const FwdParams& p, int d, bool causal, hipStream_t s) {
  if (d == 128) return launch<128, 64, false, true>(p, causal, s);
  return launch<64, 64, false, true>(p, causal, s);
}

}  // namespace fa
