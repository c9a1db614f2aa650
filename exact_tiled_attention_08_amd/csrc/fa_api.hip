// C ABI of libfa.so: argument validation, then dispatch to the HIP launchers.
// Validation makes no HIP call, so a rejected call launches and writes nothing.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr long long kMaxHeadElems = 1LL << 30;  // Nk * d per head: 32-bit in-head offsets

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// hipError_t of the most recent failed launch on this thread (hipSuccess if none).
thread_local hipError_t g_last_hip_error = hipSuccess;

fa_status finish_launch(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = e;
  return FA_ERR_HIP;
}

// (b, h) pairs handled together on one XCD (see fa::map_block). The XCD's CUs walk the
// group's query tiles together, so each K/V tile is fetched into its L2 once per round of
// concurrently running tiles of a head; with long sequences (many query tiles) fewer heads
// per group mean more tiles of one head per round, hence fewer re-reads from HBM. Measured
// on the forward with 118 query tiles per head (4 heads per XCD): HBM reads 7.3 / 3.8 /
// 1.9 GB for 4 / 2 / 1 heads per group, 1132 / 1197 / 1208 TFLOP/s; with 32 query tiles
// the order reverses (1066 / 1060 / 1039 TFLOP/s for 4 / 2 / 1 heads, though 1 head
// halves the reads), so all of the XCD's heads form one group there.
int heads_per_group(int BH, long long nqt) {
  if (BH % 8 != 0) return 1;
  const int per_xcd = BH / 8;
  return nqt > 64 ? 1 : per_xcd;
}

// Dynamic tail of a causal block map (fa::map_block_tail) over BH * nt tiles, hpg pairs
// per XCD group, tiles in descending (desc) or ascending index order within a group;
// weight(tile) is the tile's work in key or query tiles. Every XCD's run issues its tiles
// heaviest first; its trailing items whose weight (plus two for the fixed part of a
// workgroup) adds up to about kTailShare of the run's weight go to the shared pool, and
// the grid gets kTailDraws ticket-drawing blocks per pool item, so an XCD that finishes
// early can take up to that many times its share. Left off (draws = 0) when the runs are
// not alike (BH not a multiple of 8) or hold fewer than two items per CU (32 CUs per XCD).
// Measured on the bfloat16 prefill against the fixed map (bitwise-identical results):
// +1.6% at N = 8192 and +2.3% at N = 30000 on one box, +0% and +2.9% on another (the gain
// follows how unequal the box's XCDs run); per-CU busy time rose from 94-95% to 98%.
// Non-causal launches (equal tiles, two per CU on the d = 64 shape) measured -1%, so they
// keep the fixed map.
constexpr double kTailShare = 0.08;
constexpr double kTailDraws = 2.0;
std::atomic<unsigned> g_tail_seq{0};

template <typename Weight>
fa::TailMap tail_map(int BH, int nt, int hpg, bool desc, Weight weight) {
  fa::TailMap tm{};
  if (BH % 8 != 0) return tm;
  const long long per = (long long)BH * nt / 8;
  if (per < 64) return tm;
  // weight of run position t (run 0; all runs follow the same tile order)
  auto at = [&](long long t) {
    const long long j = t % ((long long)hpg * nt);
    const int i = (int)(j / hpg);
    return weight(desc ? nt - 1 - i : i) + 2;
  };
  double total = 0;
  for (long long t = 0; t < per; ++t) total += (double)at(t);
  long long pool = 0;
  double acc = 0;
  while (pool < per && acc < kTailShare * total) acc += (double)at(per - 1 - pool++);
  if (pool == 0 || pool == per) return tm;
  if (8 * per + 8 * (long long)(pool * kTailDraws) > INT32_MAX) return tm;  // grid size
  tm.per = (int)per;
  tm.s = (int)(per - pool);
  tm.pool = (int)pool;
  tm.draws = (int)(8 * pool * kTailDraws);
  return tm;
}

int tail_slot() { return (int)(g_tail_seq.fetch_add(1, std::memory_order_relaxed) % fa::kTailSlots); }

// Causal prefill: key tiles of bc keys that query tile qt (br rows) sees.
fa::TailMap prefill_tail(const fa::FwdParams& p, int br, int bc) {
  return tail_map(p.BH, p.nqt, p.hpg, true, [&](int qt) {
    const long long last_q = std::min((long long)(qt + 1) * br, (long long)p.Nq) - 1;
    const long long kv_end = std::min((long long)p.Nk, last_q + p.off + 1);
    return kv_end > 0 ? (kv_end + bc - 1) / bc : 0;
  });
}

// Causal backward: dK/dV tile kt is seen by the queries from max(0, kt*rows - off) on
// (in tiles of rows queries); dQ tile qt sees the keys up to its last row + off.
void backward_tails(fa::BwdParams& p) {
  const int rk = fa::kBwdKeyRows, rq = fa::kBwdQueryRows;
  p.tail_kv = tail_map(p.BH, p.nkt, p.hpg_kv, false, [&](int kt) {
    const long long q_first = std::max(0LL, (long long)kt * rk - p.off);
    return q_first < p.Nq ? (p.Nq - q_first + rq - 1) / rq : 0;
  });
  p.tail_q = tail_map(p.BH, p.nqt, p.hpg_q, true, [&](int qt) {
    const long long last_q = std::min((long long)(qt + 1) * rq, (long long)p.Nq) - 1;
    const long long kv_end = std::min((long long)p.Nk, last_q + p.off + 1);
    return kv_end > 0 ? (kv_end + rk - 1) / rk : 0;
  });
  p.slot_kv = tail_slot();
  p.slot_q = tail_slot();
}

// Key position of query row 0 under the causal mask: the queries are the last Nq positions
// of the key sequence (causal = 1, bottom-right) or the first Nq (causal = 2, top-left).
int query_offset(int causal, int Nq, int Nk) { return causal == 2 ? 0 : Nk - Nq; }

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "a size is < 1 or the sizes overflow the index range";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension, dtype or size";
    case FA_ERR_WORKSPACE: return "workspace is NULL or too small";
    case FA_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FA_ERR_VALUE: return "scale must be finite and > 0; causal must be 0, 1 or 2";
    case FA_ERR_ALIGN: return "a tensor pointer (or a bias stride) is not suitably aligned";
  }
  return "unknown status";
}

int fa_last_hip_error(void) { return (int)g_last_hip_error; }

const char* fa_last_hip_error_str(void) { return hipGetErrorString(g_last_hip_error); }

fa_status fa_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || BH * (long long)Nq * d > (1LL << 62) / 4) return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || (long long)Nq * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;

  const int br = dtype == FA_BF16 ? fa::fwd_bf16_block_rows(d) : fa::fwd_f32_block_rows(d);
  const long long nqt = (Nq + br - 1) / br;
  if (BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.Nq = Nq;
  p.Nk = Nk;
  p.off = query_offset(causal, Nq, Nk);
  p.nqt = (int)nqt;
  p.hpg = heads_per_group((int)BH, nqt);
  p.c = scale * fa::kLog2e;
  if (dtype == FA_BF16 && causal != 0) {
    p.tail = prefill_tail(p, br, fa::fwd_bf16_key_tile(d));
    p.tail_slot = tail_slot();
  }
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(p, d, causal != 0, (hipStream_t)stream)
                                  : fa::launch_fwd_f32(p, d, causal != 0, (hipStream_t)stream);
  return finish_launch(e);
}

fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      float* o, float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                      int causal, fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !bias) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || BH * (long long)Nq * d > (1LL << 62) / 4) return FA_ERR_SHAPE;
  if (bias_stride_b < 0 || bias_stride_h < 0 || bias_stride_q < 0) return FA_ERR_SHAPE;
  // 64-bit element offsets of the farthest bias row stay far from overflow
  const long long lim = (1LL << 62) / 4;
  if (bias_stride_b > lim / B || bias_stride_h > lim / H || bias_stride_q > lim / Nq)
    return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || (long long)Nq * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  // the bias of one wave's 32 query rows is addressed with 32-bit byte offsets
  if (bias_stride_q * 64 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  if (dtype == FA_BF16) {
    if (!aligned16(bias) || (bias_stride_b | bias_stride_h | bias_stride_q) % 8 != 0)
      return FA_ERR_ALIGN;
  } else if (((uintptr_t)bias & 3u) != 0) {
    return FA_ERR_ALIGN;
  }

  const int br = dtype == FA_BF16 ? fa::fwd_bf16_block_rows(d) : fa::fwd_f32_block_rows(d);
  const long long nqt = (Nq + br - 1) / br;
  if (BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.Nq = Nq;
  p.Nk = Nk;
  p.off = query_offset(causal, Nq, Nk);
  p.nqt = (int)nqt;
  p.hpg = heads_per_group((int)BH, nqt);
  p.c = scale * fa::kLog2e;
  p.scale = scale;
  p.H = H;
  p.bias = bias;
  p.bsb = bias_stride_b;
  p.bsh = bias_stride_h;
  p.bsq = bias_stride_q;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16_bias(p, d, causal != 0, (hipStream_t)stream)
                                  : fa::launch_fwd_f32_bias(p, d, causal != 0, (hipStream_t)stream);
  return finish_launch(e);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int total_q, int total_k, int max_seqlen_q, int d, float scale,
                        int causal, fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if (B < 1 || H < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || (long long)total_q * H * d > (1LL << 62) / 4) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // a K/V tile's rows must lie within 2^31 bytes of its first row (32-bit load offsets)
  if ((long long)H * d * 2 * 128 > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)cu_seqlens_q & 3u) != 0 || ((uintptr_t)cu_seqlens_k & 3u) != 0)
    return FA_ERR_ALIGN;
  const int br = fa::fwd_bf16_block_rows(d);
  const long long nqt = (max_seqlen_q + br - 1) / br;
  if (BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.nqt = (int)nqt;
  // One (b, h) pair per XCD group: the XCD's CUs work through one pair's query tiles
  // together and share its K/V in L2 (measured on a mix of 16 causal sequences of 330 to
  // 7117 tokens: 951 TFLOP/s against 656 with the dense heuristic's 32 pairs per group,
  // whose concurrently running tiles belong to different pairs).
  p.hpg = 1;
  p.c = scale * fa::kLog2e;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.B = B;
  p.H = H;
  p.total_q = total_q;
  p.total_k = total_k;
  p.top_left = causal == 2;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  return finish_launch(fa::launch_fwd_bf16_varlen(p, d, causal != 0, (hipStream_t)stream));
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float* o, float* lse,
                     int B, int H, int Nq, int Nk, int d, float scale, float q_descale,
                     float k_descale, float v_descale, int causal, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || BH * (long long)Nq * d > (1LL << 62) / 4) return FA_ERR_SHAPE;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || (long long)Nq * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  if (!(q_descale > 0.f) || !isfinite(q_descale) || !(k_descale > 0.f) || !isfinite(k_descale) ||
      !(v_descale > 0.f) || !isfinite(v_descale))
    return FA_ERR_VALUE;
  const float c = scale * q_descale * k_descale * fa::kLog2e;
  if (!isfinite(c) || !(c > 0.f)) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  const int br = fa::fwd_fp8_block_rows();
  const long long nqt = (Nq + br - 1) / br;
  if (BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.Nq = Nq;
  p.Nk = Nk;
  p.off = query_offset(causal, Nq, Nk);
  p.nqt = (int)nqt;
  p.hpg = heads_per_group((int)BH, nqt);
  p.c = c;
  if (causal != 0) {
    p.tail = prefill_tail(p, br, fa::fwd_fp8_key_tile());
    p.tail_slot = tail_slot();
  }
  p.vscale = v_descale;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  return finish_launch(fa::launch_fwd_fp8(p, causal != 0, (hipStream_t)stream));
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || d < 1 || num_splits < 1) return 0;
  const unsigned long long n = (unsigned long long)B * H * num_splits;
  const unsigned long long per = (unsigned long long)(d + 2) * 4ull;
  if (n > (1ull << 62) / per) return 0;
  return (size_t)(n * per);
}

fa_status fa_decode_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                            int B, int H, int Nk, int d, float scale, int num_splits,
                            void* workspace, size_t workspace_bytes, fa_dtype dtype,
                            void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nk < 1 || d < 1 || num_splits < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH * num_splits > INT32_MAX) return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || num_splits > fa::kMaxSplits) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_VALUE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace))
    return FA_ERR_ALIGN;

  fa::DecodeParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.Nk = Nk;
  p.S = num_splits;
  p.chunk = (Nk + num_splits - 1) / num_splits;
  p.c = scale * fa::kLog2e;
  // workspace: partial sums o [BH][S][d], then partial (m, l) [BH][S][2]
  p.ws_o = (float*)workspace;
  p.ws_ml = p.ws_o + (size_t)BH * num_splits * d;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  hipError_t e = fa::launch_decode(p, d, dtype == FA_BF16, (hipStream_t)stream);
  return finish_launch(e);
}

fa_status fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, float* o,
                                    float* lse, int B, int H, int Nk, int d, float scale,
                                    int num_splits, fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nk < 1 || d < 1 || num_splits < 1) return FA_ERR_SHAPE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (need == 0 || need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  // the device the work runs on: the stream's (the current one for the null stream)
  int device = -1;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return finish_launch(e);
  void* ws = nullptr;
  if ((e = fa::decode_scratch(device, &ws)) != hipSuccess) return finish_launch(e);
  return fa_decode_splitkv(q, k, v, o, lse, B, H, Nk, d, scale, num_splits, ws,
                           (size_t)FA_NOALLOC_SCRATCH_BYTES, dtype, stream);
}

fa_status fa_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                          const int* block_table, const int* seq_lens, float* o, float* lse,
                          int B, int H, int d, int page_size, int num_pages, int max_pages_per_seq,
                          float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          fa_dtype dtype, void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return FA_ERR_NULL;
  if (B < 1 || H < 1 || d < 1 || num_splits < 1 || page_size < 1 || num_pages < 1 ||
      max_pages_per_seq < 1)
    return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH * num_splits > INT32_MAX || (long long)max_pages_per_seq * page_size > INT32_MAX)
    return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((page_size & (page_size - 1)) != 0 || num_splits > fa::kMaxSplits) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_VALUE;
  const size_t need = fa_decode_workspace_bytes(B, H, d, num_splits);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(workspace) || ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seq_lens & 3u) != 0)
    return FA_ERR_ALIGN;

  fa::DecodeParams p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o = o;
  p.lse = lse;
  p.BH = (int)BH;
  p.Nk = 0;     // per sequence: seq_lens
  p.S = num_splits;
  p.chunk = 0;  // per sequence: ceil(seq_lens[b] / S)
  p.c = scale * fa::kLog2e;
  p.ws_o = (float*)workspace;
  p.ws_ml = p.ws_o + (size_t)BH * num_splits * d;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.H = H;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  p.page_shift = shift;
  p.max_pages = max_pages_per_seq;
  p.num_pages = num_pages;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  return finish_launch(fa::launch_decode_paged(p, d, dtype == FA_BF16, (hipStream_t)stream));
}

size_t fa_bwd_workspace_bytes(int B, int H, int Nq) {
  if (B < 1 || H < 1 || Nq < 1) return 0;
  const unsigned long long pad = ((unsigned long long)Nq + fa::kBwdQueryRows - 1) / fa::kBwdQueryRows *
                                 fa::kBwdQueryRows;
  const unsigned long long n = (unsigned long long)B * H * pad;
  if (n > (1ull << 60) / 8ull) return 0;
  return (size_t)(n * 8ull);  // two float32 statistics per (padded) query row
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
                 const void* dout, float* dq, float* dk, float* dv, int B, int H, int Nq, int Nk,
                 int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                 fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX) return FA_ERR_SHAPE;
  if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || (long long)Nq * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      ((uintptr_t)lse & 3u) != 0)
    return FA_ERR_ALIGN;
  const long long nkt = (Nk + fa::kBwdKeyRows - 1) / fa::kBwdKeyRows;
  const long long nqt = (Nq + fa::kBwdQueryRows - 1) / fa::kBwdQueryRows;
  if (BH * nkt > INT32_MAX || BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws = (float*)workspace;
  p.BH = (int)BH;
  p.Nq = Nq;
  p.Nk = Nk;
  p.Nq_pad = (int)(nqt * fa::kBwdQueryRows);
  p.off = query_offset(causal, Nq, Nk);
  p.nkt = (int)nkt;
  p.nqt = (int)nqt;
  p.hpg_kv = heads_per_group((int)BH, nkt);
  p.hpg_q = heads_per_group((int)BH, nqt);
  p.scale = scale;
  p.c = scale * fa::kLog2e;
  if (dtype == FA_BF16 && causal != 0) backward_tails(p);
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  if (dtype == FA_F32) return finish_launch(fa::launch_bwd_f32(p, d, causal != 0, (hipStream_t)stream));
  return finish_launch(fa::launch_bwd(p, d, causal != 0, (hipStream_t)stream));
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const float* o,
                        const float* lse, const void* dout, float* dq, float* dk, float* dv,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int H,
                        int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes,
                        fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens_q ||
      !cu_seqlens_k)
    return FA_ERR_NULL;
  if (B < 1 || H < 1 || total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
      d < 1)
    return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX || (long long)total_q * H * d > (1LL << 62) / 4 ||
      (long long)total_k * H * d > (1LL << 62) / 4)
    return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // a tile's rows must lie within 2^31 bytes of its first row (32-bit load offsets)
  if ((long long)H * d * 2 * 128 > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  const size_t need = fa_bwd_workspace_bytes(B, H, max_seqlen_q);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      ((uintptr_t)lse & 3u) != 0 || ((uintptr_t)cu_seqlens_q & 3u) != 0 ||
      ((uintptr_t)cu_seqlens_k & 3u) != 0)
    return FA_ERR_ALIGN;
  const long long nkt = (max_seqlen_k + fa::kBwdKeyRows - 1) / fa::kBwdKeyRows;
  const long long nqt = (max_seqlen_q + fa::kBwdQueryRows - 1) / fa::kBwdQueryRows;
  if (BH * nkt > INT32_MAX || BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws = (float*)workspace;
  p.BH = (int)BH;
  p.Nq = max_seqlen_q;
  p.Nk = max_seqlen_k;
  p.Nq_pad = (int)(nqt * fa::kBwdQueryRows);
  p.nkt = (int)nkt;
  p.nqt = (int)nqt;
  // one (b, h) pair per XCD group, as in the forward over packed batches
  p.hpg_kv = 1;
  p.hpg_q = 1;
  p.scale = scale;
  p.c = scale * fa::kLog2e;
  p.H = H;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.B = B;
  p.total_q = total_q;
  p.total_k = total_k;
  p.top_left = causal == 2;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  return finish_launch(fa::launch_bwd_varlen(p, d, causal != 0, (hipStream_t)stream));
}

fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const void* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      const float* o, const float* lse, const void* dout, float* dq, float* dk,
                      float* dv, float* dbias, int B, int H, int Nq, int Nk, int d, float scale,
                      int causal, void* workspace, size_t workspace_bytes, fa_dtype dtype,
                      void* stream) {
  if (!q || !k || !v || !bias || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_SHAPE;
  const long long BH = (long long)B * H;
  if (BH > INT32_MAX) return FA_ERR_SHAPE;
  if (bias_stride_b < 0 || bias_stride_h < 0 || bias_stride_q < 0) return FA_ERR_SHAPE;
  const long long lim = (1LL << 62) / 4;
  if (bias_stride_b > lim / B || bias_stride_h > lim / H || bias_stride_q > lim / Nq)
    return FA_ERR_SHAPE;
  if (dbias && BH * (long long)Nq > lim / Nk) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)Nk * d > kMaxHeadElems || (long long)Nq * d > kMaxHeadElems) return FA_ERR_UNSUPPORTED;
  // the bias rows of one 64-query tile are addressed with 32-bit byte offsets
  if (bias_stride_q * 128 >= (1LL << 31)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale) || causal < 0 || causal > 2) return FA_ERR_VALUE;
  const size_t need = fa_bwd_workspace_bytes(B, H, Nq);
  if (!workspace || need == 0 || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace) ||
      !aligned16(bias) || (dbias && !aligned16(dbias)) || ((uintptr_t)lse & 3u) != 0 ||
      (bias_stride_b | bias_stride_h | bias_stride_q) % 8 != 0)
    return FA_ERR_ALIGN;
  const long long nkt = (Nk + fa::kBwdKeyRows - 1) / fa::kBwdKeyRows;
  const long long nqt = (Nq + fa::kBwdQueryRows - 1) / fa::kBwdQueryRows;
  if (BH * nkt > INT32_MAX || BH * nqt > INT32_MAX) return FA_ERR_SHAPE;

  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.ws = (float*)workspace;
  p.BH = (int)BH;
  p.Nq = Nq;
  p.Nk = Nk;
  p.Nq_pad = (int)(nqt * fa::kBwdQueryRows);
  p.off = query_offset(causal, Nq, Nk);
  p.nkt = (int)nkt;
  p.nqt = (int)nqt;
  p.hpg_kv = heads_per_group((int)BH, nkt);
  p.hpg_q = heads_per_group((int)BH, nqt);
  p.scale = scale;
  p.c = scale * fa::kLog2e;
  p.bias = bias;
  p.bsb = bias_stride_b;
  p.bsh = bias_stride_h;
  p.bsq = bias_stride_q;
  p.H = H;
  p.dbias = dbias;
  (void)hipGetLastError();  // drop a stale error left by unrelated work on this thread
  return finish_launch(fa::launch_bwd_bias(p, d, causal != 0, (hipStream_t)stream));
}

}  // extern "C"
