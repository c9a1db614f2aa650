// Split-KV decode: one query per (b, h) against a long key/value cache.
//
// "FlashAttention: Attention Is Limited by Memory, Not Math", section "Where it helps,
// and where it does not": a single query makes attention a matrix-vector product bound by
// streaming K and V, so the key sequence is split across the GPU and the partial results
// are merged (Flash-Decoding). Each partial is a state (m, l, o) computed against its own
// max; partials merge with the two-sided rule scale_old = exp(m_a - m_new),
// scale_new = exp(m_b - m_new) ("Flash Attention Optimization", section "The fix: tile the
// computation, never materialize the full matrix"), which returns a state of the same
// shape and therefore chains ("Handwritten Notes on Flash Attention", section "Merging two
// blocks"). Empty partials (m = -inf) are skipped ("Explain FlashAttention ...", section
// "Executable recurrence, with an empty-state policy").
//
// Kernel 1 (split): workgroup (b*H + h, split s) owns keys [s*C, min(Nk, (s+1)*C)).
//   LPK lanes share one key row (16 bytes each, so a wave reads whole rows, coalesced);
//   the NT/LPK lane groups of the workgroup walk the chunk's keys round-robin, each with
//   its own running (m, l, o), updated U keys at a time. At the end the groups' states
//   are merged through LDS and written to the workspace (o unnormalised, m in log2 units).
// Kernel 2 (merge): one workgroup per (b, h), thread = output dimension; merges the S
//   partials in split order (deterministic) and writes O = o/l and LSE = ln2*(m + log2 l).
//
// Paged cache (PAGED = true): the keys of sequence b live in fixed-size pages of a shared
// pool, [num_pages][page_size][H][d], found through the sequence's block table; the same
// page indirection that engines pair with split-KV decoding (same section of "FlashAttention:
// Attention Is Limited by Memory, Not Math"). Each lane looks up the page of each of its
// keys, then loads the key's row from that page; a page id outside the pool is never read
// through and its keys are skipped. Sequence lengths may differ: each sequence's keys are
// split into S chunks of its own.
#include <mutex>

#include "../../include/fa.h"

#include "fa_internal.h"

// Partial states of the allocation-free decode entry point (fa_decode_splitkv_noalloc): a
// fixed device array in place of a caller's workspace, for callers that cannot allocate
// device memory. Every GPU the library runs on holds its own copy until the process ends.
// Host code never passes this name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known
}  // namespace

hipError_t decode_scratch(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    // once per device, with that device current
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t back = hipSetDevice(current);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!addr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = addr;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

namespace {

constexpr int kNT = 256;  // threads per split workgroup
constexpr int kU = 16;    // keys per lane group per step (loads in flight per thread: 2*kU)
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bfloat16 storage
  static constexpr int VEC = 8;
  __device__ static __forceinline__ void widen(const uint4& x, float* f) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Elem<float> {
  static constexpr int VEC = 4;
  __device__ static __forceinline__ void widen(const uint4& x, float* f) {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z);
    f[3] = __uint_as_float(x.w);
  }
};

template <int D, typename E, bool PAGED>
__global__ __launch_bounds__(kNT) void decode_split_kernel(DecodeParams p) {
  constexpr int VEC = Elem<E>::VEC;
  constexpr int LPK = D / VEC;    // lanes per key row
  constexpr int KPI = kNT / LPK;  // lane groups (keys in flight per step)
  static_assert(LPK <= 64 && (64 % LPK) == 0, "a key row must sit inside one wave");
  __shared__ float sm_ml[KPI][2];
  __shared__ float sm_o[KPI][D];

  const int tid = threadIdx.x;
  const int sub = tid % LPK;  // which 16-byte slice of the row
  const int grp = tid / LPK;  // which lane group
  const int sidx = blockIdx.x % p.S;
  const int bh = blockIdx.x / p.S;
  int len = p.Nk, chunk = p.chunk;
  const E* __restrict__ kh;
  const E* __restrict__ vh;
  const int* __restrict__ tab = nullptr;
  if (PAGED) {
    const int b = bh / p.H;
    const int h = bh - b * p.H;
    len = min(max(p.seq_lens[b], 0), p.max_pages << p.page_shift);
    chunk = (len + p.S - 1) / p.S;
    kh = (const E*)p.k + (size_t)h * D;  // row r of the pool: + r * H * D
    vh = (const E*)p.v + (size_t)h * D;
    tab = p.block_table + (size_t)b * p.max_pages;
  } else {
    kh = (const E*)p.k + (size_t)bh * p.Nk * D;
    vh = (const E*)p.v + (size_t)bh * p.Nk * D;
  }
  const int lo = sidx * chunk;
  const int hi = min(len, lo + chunk);
  float qv[VEC];
  Elem<E>::widen(*(const uint4*)((const E*)p.q + (size_t)bh * D + sub * VEC), qv);

  float m = -INFINITY, l = 0.f;
  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.f;

  // every thread runs the same trip count; a group's kU keys are base + u*KPI + grp
  for (int base = lo; base < hi; base += KPI * kU) {
    uint4 kx[kU], vx[kU];
    bool ok[kU];
    size_t row[kU];  // element offset of the key's row from kh / vh
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int key = base + u * KPI + grp;
      ok[u] = key < hi;
      if (PAGED) {
        const int page = ok[u] ? tab[key >> p.page_shift] : 0;
        ok[u] = ok[u] && (unsigned)page < (unsigned)p.num_pages;
        const size_t r = ((size_t)page << p.page_shift) | (size_t)(key & ((1 << p.page_shift) - 1));
        row[u] = r * (size_t)p.H * D;
      } else {
        row[u] = (size_t)key * D;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ok[u]) {
        // streamed once: non-temporal loads keep the cache for the workspace and q
        const v4u a = __builtin_nontemporal_load((const v4u*)(kh + row[u] + sub * VEC));
        const v4u b = __builtin_nontemporal_load((const v4u*)(vh + row[u] + sub * VEC));
        kx[u] = make_uint4(a[0], a[1], a[2], a[3]);
        vx[u] = make_uint4(b[0], b[1], b[2], b[3]);
      } else {
        kx[u] = make_uint4(0, 0, 0, 0);
        vx[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float kf[VEC];
      Elem<E>::widen(kx[u], kf);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc = __builtin_fmaf(qv[e], kf[e], acc);
      s[u] = acc;
    }
    // sum the partial dot products of the LPK lanes that share a key row
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1)
#pragma unroll
      for (int u = 0; u < kU; ++u) s[u] += __shfl_xor(s[u], off);
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      s[u] = ok[u] ? s[u] * p.c : -INFINITY;
      bm = fmaxf(bm, s[u]);
    }
    const float m_new = fmaxf(m, bm);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float pu = __builtin_amdgcn_exp2f(s[u] - m_use);
      l += pu;
      float vf[VEC];
      Elem<E>::widen(vx[u], vf);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = __builtin_fmaf(pu, vf[e], o[e]);
    }
  }

  // merge the KPI lane-group states of this chunk
  if (sub == 0) {
    sm_ml[grp][0] = m;
    sm_ml[grp][1] = l;
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) sm_o[grp][sub * VEC + e] = o[e];
  __syncthreads();
  for (int dd = tid; dd < D; dd += kNT) {
    float M = -INFINITY;
    for (int gi = 0; gi < KPI; ++gi) M = fmaxf(M, sm_ml[gi][0]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int gi = 0; gi < KPI; ++gi) {
        const float mg = sm_ml[gi][0];
        if (mg == -INFINITY) continue;
        const float wgt = __builtin_amdgcn_exp2f(mg - M);
        L = __builtin_fmaf(wgt, sm_ml[gi][1], L);
        O = __builtin_fmaf(wgt, sm_o[gi][dd], O);
      }
    }
    const size_t slot = (size_t)bh * p.S + sidx;
    p.ws_o[slot * D + dd] = O;
    if (dd == 0) {
      p.ws_ml[2 * slot] = M;
      p.ws_ml[2 * slot + 1] = L;
    }
  }
}

// The S (m, l) pairs of one (b, h) are staged in LDS once; each thread then combines the
// S partials of its output dimension with independent loads in flight.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeParams p) {
  __shared__ float sml[2 * kMaxSplits];
  const int bh = blockIdx.x;
  const int dd = threadIdx.x;
  const float* ml = p.ws_ml + (size_t)bh * p.S * 2;
  const float* os = p.ws_o + (size_t)bh * p.S * D;
  for (int i = dd; i < 2 * p.S; i += D) sml[i] = ml[i];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < p.S; ++s) M = fmaxf(M, sml[2 * s]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int s = 0; s < p.S; ++s) {
      const float ms = sml[2 * s];
      // an empty chunk (m = -inf) gets weight exp2(-inf) = 0 and its o and l are 0
      const float wgt = __builtin_amdgcn_exp2f(ms - M);
      L = __builtin_fmaf(wgt, sml[2 * s + 1], L);
      O = __builtin_fmaf(wgt, os[(size_t)s * D + dd], O);
    }
  }
  p.o[(size_t)bh * D + dd] = L > 0.f ? O / L : 0.f;
  if (dd == 0 && p.lse) p.lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D, typename E, bool PAGED>
hipError_t launch(const DecodeParams& prm, hipStream_t s) {
  DecodeParams p = prm;
  hipLaunchKernelGGL((decode_split_kernel<D, E, PAGED>), dim3(p.BH * p.S), dim3(kNT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(p.BH), dim3(D), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, hipStream_t s) {
  if (bf16) return d == 128 ? launch<128, uint16_t, false>(p, s) : launch<64, uint16_t, false>(p, s);
  return d == 128 ? launch<128, float, false>(p, s) : launch<64, float, false>(p, s);
}

hipError_t launch_decode_paged(const DecodeParams& p, int d, bool bf16, hipStream_t s) {
  if (bf16) return d == 128 ? launch<128, uint16_t, true>(p, s) : launch<64, uint16_t, true>(p, s);
  return d == 128 ? launch<128, float, true>(p, s) : launch<64, float, true>(p, s);
}

}  // namespace fa
