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

// Ticket-counter slots of the dynamic tail: a call takes the next slot of a ring, so calls
// that overlap on one GPU (different streams) use different counters.
constexpr int kTailSlots = 4096;
// Dynamic tail of the block map (map_block_tail); draws == 0: the fixed map_block.
struct TailMap {
  int per;    // items per run (the grid covers 8 * per items)
  int s;      // fixed items per run
  int pool;   // pool items per run (per - s)
  int draws;  // blocks that draw a ticket: gridDim.x - 8 * s
};

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
  int off;        // key position of query row 0 for causal masking (Nk - Nq or 0)
  int nqt;        // number of query tiles per (b, h)
  int hpg;        // (b, h) pairs per XCD group for the block -> tile mapping
  float c;        // scale * log2(e): scores are exponentiated base 2 (FP8: times both descales)
  float scale;    // additive bias only: the softmax scale itself
  float vscale;   // FP8 only: the descale factor of v
  // Packed variable-length batches only: q, k, v, o are [total][H][d], lse [H][total_q];
  // sequence b owns rows cu_q[b] .. cu_q[b+1]-1 (queries) and cu_k[b] .. cu_k[b+1]-1 (keys).
  const int* cu_q;
  const int* cu_k;
  int B;
  int H;
  int total_q;
  int total_k;
  int top_left;   // causal queries at the start of each sequence's keys (else at the end)
  // Additive bias only: element (b, h, i, j) at bias[b*bsb + h*bsh + i*bsq + j], in the
  // input dtype (a stride of 0 repeats a dimension); H above gives b and h of a pair.
  const void* bias;
  long long bsb;
  long long bsh;
  long long bsq;
  // Causal bfloat16 and FP8 prefill: the dynamic tail of the block map and its
  // ticket-counter slot.
  TailMap tail;
  int tail_slot;
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
  // Paged cache only (k, v are [num_pages][page_size][H][d]): key t of sequence b sits in
  // page block_table[b][t >> page_shift], slot t & (page_size - 1); the sequence has
  // seq_lens[b] keys, split into S chunks of ceil(seq_lens[b] / S).
  const int* block_table;  // [B][max_pages]
  const int* seq_lens;     // [B]
  int H;
  int page_shift;          // log2(page_size)
  int max_pages;           // block table entries per sequence
  int num_pages;           // pages in the pool; ids outside [0, num_pages) hold no keys
};

// Arguments of the backward kernels.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const float* o;     // forward output [BH][Nq][d]
  const float* lse;   // forward log-sum-exp [BH][Nq] (natural log)
  const void* dout;   // gradient of the loss with respect to O, [BH][Nq][d]
  float* dq;
  float* dk;
  float* dv;
  // Row statistics [BH][Nq_pad / 64][2][64]: per block of 64 query rows, the 64 LSEs in
  // log2 units (+inf for rows that see no key and for padding rows, so that their
  // probabilities come out 0), then the 64 values sum_t dO[i][t] * O[i][t] (0 for padding).
  float* ws;
  int BH;
  int Nq;
  int Nk;
  int Nq_pad;         // Nq rounded up to a whole number of dQ query tiles
  int off;            // key position of query row 0 for causal masking (Nk - Nq or 0)
  int nkt;            // key tiles per (b, h) of the dK/dV kernel
  int nqt;            // query tiles per (b, h) of the dQ kernel
  int hpg_kv;         // (b, h) pairs per XCD group, dK/dV kernel
  int hpg_q;          // (b, h) pairs per XCD group, dQ kernel
  float scale;
  float c;            // scale * log2(e)
  // Additive bias only (the backward of fa_fwd_bias): element (b, h, i, j) at
  // bias[b*bsb + h*bsh + i*bsq + j] (bfloat16), H gives b and h of a pair; dbias, if not
  // null, receives dL/dbias = dS as a full float32 [B][H][Nq][Nk] tensor.
  const void* bias;
  long long bsb;
  long long bsh;
  long long bsq;
  int H;
  float* dbias;
  // Variable-length batches only (the backward of fa_fwd_varlen): q, dout, o, dq are packed
  // [total_q][H][d] and k, v, dk, dv [total_k][H][d]; lse is [H][total_q]. Pair bh = h*B + b
  // is sequence b of head h (cu_q, cu_k: B+1 device offsets, clamped into the tensors);
  // Nq and Nk above are the caps max_seqlen_q and max_seqlen_k, and every pair's workspace
  // block holds Nq_pad rows. top_left: causal alignment 2.
  const int* cu_q;
  const int* cu_k;
  int B;
  int total_q;
  int total_k;
  int top_left;
  // Causal bfloat16 backward (dense, no bias): the dynamic tails of the dK/dV and dQ block
  // maps and their ticket-counter slots.
  TailMap tail_kv;
  TailMap tail_q;
  int slot_kv;
  int slot_q;
};

// Workgroup barrier without the memory fence of __syncthreads(): the fence would also wait
// for this wave's in-flight direct-to-LDS loads, which must keep flying across the phase
// barrier. LDS reads are drained first; loads are waited for explicitly where their data
// is needed. The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory loads are still in flight (loads
// complete in issue order, so the ones issued before the last N have landed).
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One global_load_lds_dwordx4: each lane copies 16 bytes from (uniform base + its 32-bit
// byte offset) to LDS byte address lds_base + 16*lane (lds_base wave-uniform, in M0).
// Written as inline asm so that the compiler does not treat later LDS reads of OTHER
// buffers as possible readers of this copy and stall them on vmcnt; completion is awaited
// explicitly with wait_loads() before the barrier that publishes the buffer. The offset
// register is the caller's long-lived VGPR, so no later instruction overwrites it while
// the load is in flight.
//
// M0 (the LDS address of a direct load) is declared clobbered rather than saved and
// restored around each copy: two scalar instructions fewer per load in the tile bursts,
// which sit on the prefill kernels' critical path (same process, bitwise-identical
// results: +0.2% on the bf16 causal prefills, +1.4-2.2% on the FP8 prefill; one statement
// per tile with a single save and restore measured 0.5-1.6% slower, its slot bases all
// computed before the first copy). The compiler reserves M0 and would not restore a value
// of its own kept across such a statement; it never writes M0 in the kernels that use
// these helpers (none of their instructions needs M0), which a CPU test checks on their
// gfx950 assembly, so the warning about the reserved register is silenced here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory", "m0");
}

// dma16 to LDS byte address lds_base + IMM: the constant is added to M0 inside the copy, so
// the slots of one buffer need one scalar base between them (the compiler would otherwise
// keep one scalar per slot alive across the loop and spill them to vector registers).
template <int IMM>
__device__ __forceinline__ void dma16_at(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds_base), "i"(IMM)
      : "memory", "scc", "m0");
}
#pragma clang diagnostic pop

// Launchers (defined next to their kernels). Each returns the hipError_t of the launch.
hipError_t launch_fwd_bf16(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_bf16_varlen(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_bf16_bias(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_f32_bias(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_fwd_fp8(const FwdParams& p, bool causal, hipStream_t s);
int fwd_fp8_block_rows();
int fwd_fp8_key_tile();  // keys per K/V tile of the FP8 kernel
hipError_t launch_fwd_f32(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s);
hipError_t launch_decode_paged(const DecodeParams& p, int d, bool bf16, hipStream_t s);
// Device address of the decode's fixed scratch array on `device` (looked up once per device
// with hipGetSymbolAddress, then cached); FA_NOALLOC_SCRATCH_BYTES long.
hipError_t decode_scratch(int device, void** ptr);
hipError_t launch_bwd(const BwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_bias(const BwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_varlen(const BwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_bwd_f32(const BwdParams& p, int d, bool causal, hipStream_t s);

// Query rows per workgroup of each prefill kernel (host needs it for the grid).
int fwd_bf16_block_rows(int d);
int fwd_bf16_key_tile(int d);  // keys per K/V tile of fa_fwd's bfloat16 kernel
int fwd_f32_block_rows(int d);

// Stores a wave's 32 x D float32 tile of MFMA accumulators (lane column = row, element i of
// acc[db] = column 32db + 8(i/4) + 4g + i%4, g = lane / 32), each lane's values times `mul`,
// to rows 0 .. nvalid-1 of `out` (row stride rs floats). A lane holds 16-byte pieces of
// one row, so storing them directly writes 32 bytes of each of 32 rows per instruction.
// Here they pass through the wave's own 8 KB of LDS at `stage`, 64 columns at a time,
// and are read back row-major: each store then writes whole 256-byte segments of 4 rows.
// Chunk c of row r sits at chunk position c ^ (r % 16), which keeps both the writes and
// the reads free of bank conflicts. The stores are non-temporal (the outputs are written
// once and not read by the kernel; streamed past L2 they leave its K/V tiles there).
// The caller makes sure no other wave uses `stage` meanwhile. (The two prefill kernels keep
// an inline copy of these steps: through this function their code came out with other
// register assignments and measured 0.35-0.6% slower.)
template <int D>
__device__ __forceinline__ void store_rows_staged(const f32x16 (&acc)[D / 32], float mul, char* stage,
                                                  float* out, size_t rs, int nvalid, int lane) {
  const int col = lane & 31, g = lane >> 5;
#pragma unroll
  for (int hh = 0; hh < D / 64; ++hh) {
#pragma unroll
    for (int dbh = 0; dbh < 2; ++dbh)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int db = 2 * hh + dbh;
        f32x4 val;
        val[0] = acc[db][4 * j + 0] * mul;
        val[1] = acc[db][4 * j + 1] * mul;
        val[2] = acc[db][4 * j + 2] * mul;
        val[3] = acc[db][4 * j + 3] * mul;
        const int c = 8 * dbh + 2 * j + g;  // columns 64 hh + 4c .. 64 hh + 4c + 3
        *(f32x4*)(stage + col * 256 + ((c ^ (col & 15)) << 4)) = val;
      }
    asm volatile("" ::: "memory");  // one wave's LDS accesses complete in issue order
    const int c = lane & 15;
    f32x4 rd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + (lane >> 4);
      rd[i] = *(const f32x4*)(stage + r * 256 + ((c ^ (r & 15)) << 4));
    }
    float* const obase = out + (size_t)(lane >> 4) * rs + 64 * hh + 4 * c;
    if (nvalid >= 32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * rs));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (4 * i + (lane >> 4) < nvalid) __builtin_nontemporal_store(rd[i], (f32x4*)(obase + (size_t)(4 * i) * rs));
    }
    asm volatile("" ::: "memory");
  }
}

// Key rows per dK/dV workgroup and query rows per dQ workgroup of the backward pass.
constexpr int kBwdKeyRows = 128;
constexpr int kBwdQueryRows = 128;

// Block -> (b*H + h, query tile) mapping shared by the prefill kernels.
//
// Workgroups are handed to the 8 XCDs round-robin by block id, and each XCD has
// its own L2. The first 8*floor(total/8) blocks are renumbered so that XCD x
// receives one contiguous run of work items; inside a run, items walk a group of
// `hpg` heads query-tile by query-tile, so the query tiles of one head run
// together on one XCD and share its K/V in L2. For causal attention the query
// tiles are issued heaviest (most key tiles) first, which evens out the tail.
// Item n of the renumbered order -> (b*H + h, query tile).
__device__ __forceinline__ void map_item(int n, int nqt, int hpg, bool causal, int& bh, int& qt) {
  const int span = hpg * nqt;
  const int grp = n / span;
  const int j = n - grp * span;
  const int qi = j / hpg;
  qt = causal ? (nqt - 1 - qi) : qi;
  bh = grp * hpg + (j - qi * hpg);
}

__device__ __forceinline__ void map_block(int L, int total, int nqt, int hpg, bool causal,
                                          int& bh, int& qt) {
  const int per = total >> 3;
  const int n = (L < (per << 3)) ? (L & 7) * per + (L >> 3) : L;
  map_item(n, nqt, hpg, causal, bh, qt);
}

// The same map with a dynamic tail. The XCDs do not run at one speed: on the same tiles a
// whole XCD can take ~10% longer than another (per-workgroup real-time stamps; which XCDs
// are slow changes with the data's placement, not from run to run), and a fixed map ends
// when the slowest XCD does. Here the first `s` items of each XCD's run stay fixed (block
// L = 8t + x runs item t of run x, t < s); the remaining `pool` items of every run (the
// lightest ones: runs issue heaviest first) form one pool, interleaved across the runs
// so that it too is ordered heaviest first, and every later block takes the next pool
// item with one atomic increment of a ticket counter. An XCD that finishes its fixed
// items early therefore takes more of the pool. There are `draws` later blocks, more
// than pool items, so an XCD can take more than its share; a block that draws a ticket
// past the pool exits at once. Exactly `draws` tickets are drawn per launch, and the
// block that draws the last one puts the counter back to 0 for the next launch that uses
// it. `*s_item` is workgroup-shared scratch. Returns false when the block has no item.
__device__ __forceinline__ bool map_block_tail(const TailMap& tm, unsigned* tickets, int* s_item,
                                               int nqt, int hpg, bool causal, int& bh, int& qt) {
  const int L = blockIdx.x;
  const int t = L >> 3;
  int n;
  if (t < tm.s) {
    n = (L & 7) * tm.per + t;
  } else {
    if (threadIdx.x == 0) {
      const unsigned k = atomicAdd(tickets, 1u);
      if (k + 1 == (unsigned)tm.draws) atomicExch(tickets, 0u);
      *s_item = k < 8u * (unsigned)tm.pool ? (int)(k & 7) * tm.per + tm.s + (int)(k >> 3) : -1;
    }
    __syncthreads();
    n = *s_item;
    if (n < 0) return false;
  }
  map_item(n, nqt, hpg, causal, bh, qt);
  return true;
}

}  // namespace fa
