// C ABI of the CSA indexer library: argument validation, workspace sizing,
// kernel dispatch and error reporting.  Nothing here allocates device memory
// or synchronises; every launch goes to the caller's stream.
#include "../../include/csa_indexer.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "csa_internal.hpp"

namespace {

thread_local std::string g_last_error;

csa_status fail(csa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

csa_status ok() {
  g_last_error.clear();
  return CSA_OK;
}

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// A dispatch counts work-items per grid dimension in 32 bits: one workgroup
// per row of `threads` threads allows at most this many rows.
long long max_rows_per_dispatch(int threads) { return ((1ll << 32) - 1) / threads; }

// Test options (csa_set_test_option): process-wide, 0 = default behaviour.
std::atomic<long long> g_opt_force_generic{0};
std::atomic<long long> g_opt_cand_cap{0};
std::atomic<long long> g_opt_decode_chunk{0};

csa_status validate_problem(const csa_problem* p) {
  if (!p) return fail(CSA_ERR_INVALID, "problem pointer is NULL");
  if (p->struct_size != sizeof(csa_problem))
    return fail(CSA_ERR_INVALID, "struct_size %u != sizeof(csa_problem) %zu", p->struct_size,
                sizeof(csa_problem));
  if (p->dtype != CSA_BF16 && p->dtype != CSA_F32) return fail(CSA_ERR_INVALID, "unknown dtype %d", p->dtype);
  if (p->B <= 0 || p->S_q <= 0 || p->T <= 0 || p->H <= 0 || p->D <= 0)
    return fail(CSA_ERR_INVALID, "dimensions must be positive (B=%d S_q=%d T=%d H=%d D=%d)", p->B, p->S_q,
                p->T, p->H, p->D);
  if (p->m < 1) return fail(CSA_ERR_INVALID, "compression ratio m=%d < 1", p->m);
  if (p->q_pos0 < 0) return fail(CSA_ERR_INVALID, "q_pos0=%lld < 0", (long long)p->q_pos0);
  if (!p->q || !p->k || !p->w) return fail(CSA_ERR_INVALID, "q, k and w must not be NULL");
  if (p->D != 32 && p->D != 64 && p->D != 128 && p->D != 256)
    return fail(CSA_ERR_UNSUPPORTED, "D=%d not in {32,64,128,256}", p->D);
  if (p->H > CSA_MAX_HEADS) return fail(CSA_ERR_UNSUPPORTED, "H=%d > %d", p->H, CSA_MAX_HEADS);
  if ((long long)p->B * p->S_q > (1ll << 31) - 1) return fail(CSA_ERR_UNSUPPORTED, "B*S_q too large");
  return CSA_OK;
}

csa_status validate_flags(uint32_t flags) {
  if (flags & ~(uint32_t)(CSA_SORTED | CSA_NONCAUSAL)) return fail(CSA_ERR_INVALID, "unknown flag bits 0x%x", flags);
  return CSA_OK;
}

csa_status validate_k(int32_t k, const char* what) {
  if (k < 1) return fail(CSA_ERR_INVALID, "%s=%d < 1", what, k);
  if (k > CSA_MAX_TOPK) return fail(CSA_ERR_UNSUPPORTED, "%s=%d > %d", what, k, CSA_MAX_TOPK);
  return CSA_OK;
}

bool use_mfma(const csa_problem* p) {
  if (g_opt_force_generic.load(std::memory_order_relaxed)) return false;
  return p->dtype == CSA_BF16 && p->H == 64 && p->D == 128;
}

// Candidate buffer capacity per query row: the top-k plus eleven times as
// many appends between compactions (12k + 64).  The minimum that keeps
// progress is 2k + 64, but every compaction holds the MFMA kernel's whole
// workgroup at a barrier, so long rows run faster with fewer, larger ones
// (k = 2048, measured against 4k + 64: the million-token tail 27.6 -> 26.9
// ms, S=65536/T=16384 8.78 -> 8.49 ms; 16k + 64 and more are slower again, as
// the first fill offers every key).  Rows of at most 12k visible keys never
// compact.  The CSA_OPT_CAND_CAP test option overrides it (tests force
// frequent compactions); it is clamped to the minimum.
int cand_capacity(int kk) {
  const int lo = 2 * kk + 64;
  long long c = 12ll * kk + 64;
  const long long v = g_opt_cand_cap.load(std::memory_order_relaxed);
  if (v > 0) c = std::max<long long>(v, lo);
  return (int)((c + 63) / 64 * 64);
}

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  return n;
}

int occupancy_cached(int mode, bool mfma, bool bf16) {
  static std::mutex mu;
  static int cache[64][3][2][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> g(mu);
  int& c = cache[dev][mode][mfma][bf16];
  if (c == 0) c = csa::prefill_blocks_per_cu(mode, mfma, bf16);
  return c;
}

struct PrefillPlan {
  int rows, nqb, ws_slots, C;
  long long n_items;
  size_t cand_bytes, sort_bytes, total;
};

// Work items (query blocks x partitions) one prefill launch can index: the
// kernels count rounds of the persistent grid in 32-bit ints.
constexpr long long PF_MAX_ITEMS = (long long)INT_MAX - csa::PF_MAX_GRID;

// Workspace layout: [ws_slots workgroups x rows-per-block candidate buffers of C
// keys][sort scratch when CSA_SORTED].  ws_slots is the persistent grid: the
// workgroups resident on this device at once (compute units x occupancy of
// the chosen kernel), at most one per work item and at most PF_MAX_GRID.
PrefillPlan plan_prefill(const csa_problem* p, int mode, int kk, int P, int out_stride, uint32_t flags) {
  PrefillPlan pl;
  const bool mfma = use_mfma(p);
  pl.rows = csa::prefill_rows_per_block(mfma);
  pl.nqb = (p->S_q + pl.rows - 1) / pl.rows;
  const long long items = (long long)p->B * pl.nqb * P;
  pl.n_items = items;
  const long long resident = (long long)device_cus() * occupancy_cached(mode, mfma, p->dtype == CSA_BF16);
  pl.ws_slots = (int)std::min<long long>({items, std::max<long long>(1, resident), (long long)csa::PF_MAX_GRID});
  pl.C = cand_capacity(kk);
  pl.cand_bytes = align_up((size_t)pl.ws_slots * pl.rows * pl.C * sizeof(unsigned long long));
  pl.sort_bytes = (flags & CSA_SORTED) ? align_up((size_t)p->B * p->S_q * out_stride * sizeof(float)) : 0;
  pl.total = pl.cand_bytes + pl.sort_bytes;
  return pl;
}

// Decode path: bf16, H=64, D=128, few query rows.
bool decode_fast(const csa_problem* p) {
  return use_mfma(p) && p->S_q <= CSA_MAX_DECODE_SQ &&
         (long long)p->B * p->S_q <= max_rows_per_dispatch(csa::DEC_SEL_THREADS);
}

struct DecodePlan {
  int chunk, nsplit, nbw;
  size_t score_bytes, bound_bytes, sort_bytes, total;
};

// Keys per scan workgroup: 2048 where a full-length row still gives each of
// its waves a bound target of at most 64 keys (k <= T/8) and the launch still
// has two workgroups per CU of an MI355X (256 CUs); else 1024.  Measured at
// B=32, T=32768, k=2048: 61.7 -> 60.4 us per decode call.
int decode_chunk(const csa_problem* p, int kk) {
  const long long forced = g_opt_decode_chunk.load(std::memory_order_relaxed);
  if (forced == csa::DEC_CHUNK || forced == csa::DEC_CHUNK_LONG) return (int)forced;
  const long long rows = (long long)p->B * p->S_q;
  const long long wgs = rows * ((p->T + csa::DEC_CHUNK_LONG - 1) / csa::DEC_CHUNK_LONG);
  return (8ll * kk <= p->T && wgs >= 512) ? csa::DEC_CHUNK_LONG : csa::DEC_CHUNK;
}

DecodePlan plan_decode(const csa_problem* p, int kk, uint32_t flags) {
  DecodePlan d;
  d.chunk = decode_chunk(p, kk);
  d.nsplit = (p->T + d.chunk - 1) / d.chunk;
  d.nbw = d.nsplit * (csa::DEC_THREADS / 64);
  d.score_bytes = align_up((size_t)p->B * p->S_q * csa::dec_row_floats(p->T) * sizeof(float));
  d.bound_bytes = align_up((size_t)p->B * p->S_q * d.nbw * sizeof(uint4));
  d.sort_bytes = (flags & CSA_SORTED) ? align_up((size_t)p->B * p->S_q * kk * sizeof(float)) : 0;
  d.total = d.score_bytes + d.bound_bytes + d.sort_bytes;
  return d;
}

csa_status run_prefill_family(const csa_problem* p, int mode, int kk, int P, uint32_t flags,
                              unsigned long long thr_fixed, int32_t* out_idx, float* out_score,
                              int32_t* out_count, void* ws, size_t ws_bytes, void* stream) {
  const int out_stride = kk * P;
  const PrefillPlan pl = plan_prefill(p, mode, kk, P, out_stride, flags);
  if (pl.n_items > PF_MAX_ITEMS)
    return fail(CSA_ERR_UNSUPPORTED, "B * ceil(S_q/%d) * P = %lld query blocks above %lld per call", pl.rows,
                pl.n_items, PF_MAX_ITEMS);
  const bool sorted = (flags & CSA_SORTED) != 0;
  const long long sort_rows = (long long)p->B * p->S_q * P;     // one sort workgroup per output row segment
  if (sorted && sort_rows > max_rows_per_dispatch(256))
    return fail(CSA_ERR_UNSUPPORTED, "CSA_SORTED supports at most %lld output rows (B*S_q*P = %lld)",
                max_rows_per_dispatch(256), sort_rows);
  if (ws_bytes < pl.total || (pl.total > 0 && !ws))
    return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, pl.total);
  if ((uintptr_t)ws % 16) return fail(CSA_ERR_INVALID, "workspace must be 16-byte aligned");
  const bool mfma = use_mfma(p);
  float* score_dst = out_score;
  if (sorted && !score_dst) score_dst = (float*)((char*)ws + pl.cand_bytes);

  csa::PrefillArgs a{};
  a.q = p->q; a.k = p->k; a.w = p->w; a.kv_len = p->kv_len;
  a.B = p->B; a.S_q = p->S_q; a.T = p->T; a.H = p->H; a.D = p->D; a.m = p->m;
  a.q_pos0 = p->q_pos0;
  a.causal = (flags & CSA_NONCAUSAL) ? 0 : 1;
  a.kk = kk; a.P = P; a.nqb = pl.nqb; a.n_items = (int)pl.n_items;
  a.thr_fixed = thr_fixed;
  a.out_idx = out_idx; a.out_score = score_dst; a.out_count = out_count;
  a.out_stride = out_stride;
  a.cand = (unsigned long long*)ws;
  a.C = pl.C;
  a.need_scores = score_dst != nullptr;
  a.bf16 = p->dtype == CSA_BF16;

  const int grid = std::max(1, pl.ws_slots);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = csa::launch_prefill(a, mode, mfma, grid, st);
  if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "prefill launch failed: %s", hipGetErrorString(e));
  if (sorted) {
    e = csa::launch_sort_rows(out_idx, score_dst, sort_rows, kk, st);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "sort launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

const char* csa_status_str(csa_status s) {
  switch (s) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID: return "CSA_ERR_INVALID: invalid argument";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: shape or parameter not supported by this library version";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace too small";
    case CSA_ERR_DEVICE: return "CSA_ERR_DEVICE: HIP runtime or launch failure";
  }
  return "unknown csa_status";
}

const char* csa_last_error(void) { return g_last_error.c_str(); }

csa_status csa_set_test_option(int32_t option, int64_t value) {
  switch (option) {
    case CSA_OPT_FORCE_GENERIC:
      if (value != 0 && value != 1) return fail(CSA_ERR_INVALID, "CSA_OPT_FORCE_GENERIC takes 0 or 1");
      g_opt_force_generic.store(value);
      return ok();
    case CSA_OPT_CAND_CAP:
      if (value < 0 || value > (1ll << 30)) return fail(CSA_ERR_INVALID, "CSA_OPT_CAND_CAP outside [0, 2^30]");
      g_opt_cand_cap.store(value);
      return ok();
    case CSA_OPT_DECODE_CHUNK:
      if (value != 0 && value != csa::DEC_CHUNK && value != csa::DEC_CHUNK_LONG)
        return fail(CSA_ERR_INVALID, "CSA_OPT_DECODE_CHUNK takes 0, %d or %d", csa::DEC_CHUNK, csa::DEC_CHUNK_LONG);
      g_opt_decode_chunk.store(value);
      return ok();
  }
  return fail(CSA_ERR_INVALID, "unknown test option %d", option);
}

int csa_version(void) { return 100; }   // 0.1.0

csa_status csa_workspace_size(int op, const csa_problem* prob, int32_t k_or_cap, int32_t P, uint32_t flags,
                              size_t* bytes) {
  try {
    if (!bytes) return fail(CSA_ERR_INVALID, "bytes pointer is NULL");
    *bytes = 0;
    if (op == CSA_OP_RECALL) return ok();
    if (op < CSA_OP_PREFILL || op > CSA_OP_INTERLEAVED) return fail(CSA_ERR_INVALID, "unknown op %d", op);
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(k_or_cap, "k")) != CSA_OK) return s;
    int parts = 1;
    if (op == CSA_OP_INTERLEAVED) {
      if (P < 1) return fail(CSA_ERR_INVALID, "P=%d < 1", P);
      if ((long long)P * k_or_cap > (1ll << 30)) return fail(CSA_ERR_UNSUPPORTED, "P*k_local too large");
      parts = P;
    }
    if (op == CSA_OP_DECODE && prob->S_q > CSA_MAX_DECODE_SQ)
      return fail(CSA_ERR_UNSUPPORTED, "decode needs S_q <= %d", CSA_MAX_DECODE_SQ);
    if ((op == CSA_OP_DECODE || op == CSA_OP_THRESHOLD) && decode_fast(prob)) {
      *bytes = plan_decode(prob, k_or_cap, flags).total;
    } else {
      const int mode = op == CSA_OP_THRESHOLD     ? csa::MODE_THRESHOLD
                       : op == CSA_OP_INTERLEAVED ? csa::MODE_INTERLEAVED
                                                  : csa::MODE_TOPK;
      *bytes = plan_prefill(prob, mode, k_or_cap, parts, k_or_cap * parts, flags).total;
    }
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

}  // extern "C"

namespace {

// sigma(I + bias) > tau  <=>  I > theta = log(tau/(1-tau)) - bias, decided on the
// fp32 score: I > theta  <=>  I >= f, f = the smallest float above theta; the
// selection key of f with any index is the smallest surviving key.
unsigned long long threshold_key(float prob_threshold, float logit_bias) {
  const double t = (double)prob_threshold;
  const double theta = std::log(t / (1.0 - t)) - (double)logit_bias;
  float f = (float)theta;
  if ((double)f <= theta) f = std::nextafter(f, INFINITY);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if (u == 0x80000000u) u = 0u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (unsigned long long)ord << 32;
}

// Decode-shaped problems (bf16, H=64, D=128, S_q <= CSA_MAX_DECODE_SQ): the
// key scan, then the per-row select; thr != 0 selects threshold mode
// (survivors = keys >= thr, counted into out_count, the best kk written).
csa_status run_decode(const csa_problem* prob, int kk, uint32_t flags, unsigned long long thr, int32_t* out_idx,
                      float* out_score, int32_t* out_count, void* ws, size_t ws_bytes, void* hip_stream) {
  const DecodePlan d = plan_decode(prob, kk, flags);
  if (ws_bytes < d.total || !ws) return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, d.total);
  if ((uintptr_t)ws % 16) return fail(CSA_ERR_INVALID, "workspace must be 16-byte aligned");
  const bool sorted = (flags & CSA_SORTED) != 0;
  float* score_dst = out_score;
  if (sorted && !score_dst) score_dst = (float*)((char*)ws + d.score_bytes + d.bound_bytes);
  csa::DecodeArgs a{};
  a.q = prob->q; a.k = prob->k; a.w = prob->w; a.kv_len = prob->kv_len;
  a.B = prob->B; a.S_q = prob->S_q; a.T = prob->T; a.m = prob->m; a.q_pos0 = prob->q_pos0;
  a.causal = (flags & CSA_NONCAUSAL) ? 0 : 1;
  a.thr_fixed = thr;
  a.out_count = out_count;
  a.scores = (float*)ws;
  a.bounds = (uint4*)((char*)ws + d.score_bytes);
  a.nbw = d.nbw;
  a.chunk = d.chunk;
  a.kk = kk;
  a.out_idx = out_idx;
  a.out_score = score_dst;
  hipStream_t st = (hipStream_t)hip_stream;
  hipError_t e = csa::launch_decode(a, d.nsplit, st);
  if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
  if (sorted) {
    e = csa::launch_sort_rows(out_idx, score_dst, (long long)prob->B * prob->S_q, kk, st);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "sort launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

csa_status csa_index_topk_prefill(const csa_problem* prob, int32_t topk, uint32_t flags, int32_t* out_idx,
                                  float* out_score, void* ws, size_t ws_bytes, void* hip_stream) {
  try {
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(topk, "topk")) != CSA_OK) return s;
    if (!out_idx) return fail(CSA_ERR_INVALID, "out_idx is NULL");
    return run_prefill_family(prob, csa::MODE_TOPK, topk, 1, flags, 0ull, out_idx, out_score, nullptr, ws,
                              ws_bytes, hip_stream);
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_index_topk_decode(const csa_problem* prob, int32_t topk, uint32_t flags, int32_t* out_idx,
                                 float* out_score, void* ws, size_t ws_bytes, void* hip_stream) {
  try {
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(topk, "topk")) != CSA_OK) return s;
    if (!out_idx) return fail(CSA_ERR_INVALID, "out_idx is NULL");
    if (prob->S_q > CSA_MAX_DECODE_SQ)
      return fail(CSA_ERR_UNSUPPORTED, "decode needs S_q <= %d (got %d)", CSA_MAX_DECODE_SQ, prob->S_q);
    if (!decode_fast(prob))
      return run_prefill_family(prob, csa::MODE_TOPK, topk, 1, flags, 0ull, out_idx, out_score, nullptr, ws,
                                ws_bytes, hip_stream);
    return run_decode(prob, topk, flags, 0ull, out_idx, out_score, nullptr, ws, ws_bytes, hip_stream);
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_index_topk_decode_noalloc(const csa_problem* prob, int32_t topk, uint32_t flags, int32_t* out_idx,
                                         float* out_score, void* hip_stream) {
  try {
    static_assert(CSA_NOALLOC_SCRATCH_BYTES == csa::NOALLOC_SCRATCH_BYTES, "scratch size");
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(topk, "topk")) != CSA_OK) return s;
    if (!out_idx) return fail(CSA_ERR_INVALID, "out_idx is NULL");
    if (prob->S_q > CSA_MAX_DECODE_SQ)
      return fail(CSA_ERR_UNSUPPORTED, "decode needs S_q <= %d (got %d)", CSA_MAX_DECODE_SQ, prob->S_q);
    if (!decode_fast(prob))
      return fail(CSA_ERR_UNSUPPORTED, "the no-allocation decode needs bf16 q and k with H=64, D=128");
    const DecodePlan d = plan_decode(prob, topk, flags);
    if (d.total > csa::NOALLOC_SCRATCH_BYTES)
      return fail(CSA_ERR_UNSUPPORTED, "problem needs %zu bytes of scratch, above the %zu this entry point holds "
                  "(B*S_q*(T+67)*4 bytes of scores plus bounds); use csa_index_topk_decode with a workspace",
                  d.total, csa::NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    const hipError_t e = csa::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "scratch address lookup failed: %s", hipGetErrorString(e));
    return run_decode(prob, topk, flags, 0ull, out_idx, out_score, nullptr, ws, csa::NOALLOC_SCRATCH_BYTES, hip_stream);
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_index_threshold_select(const csa_problem* prob, float prob_threshold, float logit_bias,
                                      int32_t cap, uint32_t flags, int32_t* out_idx, int32_t* out_count,
                                      float* out_score, void* ws, size_t ws_bytes, void* hip_stream) {
  try {
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(cap, "cap")) != CSA_OK) return s;
    if (!out_idx || !out_count) return fail(CSA_ERR_INVALID, "out_idx and out_count must not be NULL");
    if (!(prob_threshold > 0.0f && prob_threshold < 1.0f))
      return fail(CSA_ERR_INVALID, "prob_threshold must be in (0,1)");
    if (!std::isfinite(logit_bias)) return fail(CSA_ERR_INVALID, "logit_bias must be finite");
    const unsigned long long thr = threshold_key(prob_threshold, logit_bias);
    if (decode_fast(prob))                            // few query rows: the decode key scan and select
      return run_decode(prob, cap, flags, thr, out_idx, out_score, out_count, ws, ws_bytes, hip_stream);
    return run_prefill_family(prob, csa::MODE_THRESHOLD, cap, 1, flags, thr, out_idx, out_score, out_count, ws,
                              ws_bytes, hip_stream);
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

static_assert(csa::DEC_MAX_BATCH == CSA_MAX_UNION_LISTS, "layer batch and union list limits agree");

csa_status csa_index_threshold_select_layers(const csa_problem* const* probs, int32_t L, float prob_threshold,
                                             float logit_bias, int32_t cap, uint32_t flags, int32_t* const* out_idx,
                                             int32_t* const* out_count, float* const* out_score, void* ws,
                                             size_t ws_bytes, void* hip_stream) {
  try {
    if (L < 1 || L > csa::DEC_MAX_BATCH) return fail(CSA_ERR_INVALID, "L=%d outside [1, %d]", L, csa::DEC_MAX_BATCH);
    if (!probs || !out_idx || !out_count) return fail(CSA_ERR_INVALID, "probs, out_idx and out_count must not be NULL");
    csa_status s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(cap, "cap")) != CSA_OK) return s;
    if (!(prob_threshold > 0.0f && prob_threshold < 1.0f))
      return fail(CSA_ERR_INVALID, "prob_threshold must be in (0,1)");
    if (!std::isfinite(logit_bias)) return fail(CSA_ERR_INVALID, "logit_bias must be finite");
    for (int i = 0; i < L; ++i) {
      if ((s = validate_problem(probs[i])) != CSA_OK) return s;
      if (!out_idx[i] || !out_count[i]) return fail(CSA_ERR_INVALID, "out_idx[%d] and out_count[%d] must not be NULL", i, i);
      if (!decode_fast(probs[i])) return fail(CSA_ERR_UNSUPPORTED, "problem %d is not decode-shaped (bf16, H=64, D=128, S_q<=%d)", i, CSA_MAX_DECODE_SQ);
      if (probs[i]->B != probs[0]->B || probs[i]->S_q != probs[0]->S_q || probs[i]->T != probs[0]->T)
        return fail(CSA_ERR_UNSUPPORTED, "problems must share B, S_q and T");
    }
    const DecodePlan d = plan_decode(probs[0], cap, flags);
    const size_t need = d.total * (size_t)L;
    if (ws_bytes < need || !ws) return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    if ((uintptr_t)ws % 16) return fail(CSA_ERR_INVALID, "workspace must be 16-byte aligned");
    const unsigned long long thr = threshold_key(prob_threshold, logit_bias);
    const bool sorted = (flags & CSA_SORTED) != 0;
    csa::DecodeBatch bt{};
    bt.L = L;
    float* score_dst[csa::DEC_MAX_BATCH];
    for (int i = 0; i < L; ++i) {
      const csa_problem* p = probs[i];
      char* wp = (char*)ws + d.total * i;
      score_dst[i] = out_score ? out_score[i] : nullptr;
      if (sorted && !score_dst[i]) score_dst[i] = (float*)(wp + d.score_bytes + d.bound_bytes);
      csa::DecodeArgs& a = bt.a[i];
      a.q = p->q; a.k = p->k; a.w = p->w; a.kv_len = p->kv_len;
      a.B = p->B; a.S_q = p->S_q; a.T = p->T; a.m = p->m; a.q_pos0 = p->q_pos0;
      a.causal = (flags & CSA_NONCAUSAL) ? 0 : 1;
      a.thr_fixed = thr;
      a.out_count = out_count[i];
      a.scores = (float*)wp;
      a.bounds = (uint4*)(wp + d.score_bytes);
      a.nbw = d.nbw;
      a.chunk = d.chunk;
      a.kk = cap;
      a.out_idx = out_idx[i];
      a.out_score = score_dst[i];
    }
    hipStream_t st = (hipStream_t)hip_stream;
    hipError_t e = csa::launch_decode_batch(bt, d.nsplit, st);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "decode launch failed: %s", hipGetErrorString(e));
    if (sorted) {
      for (int i = 0; i < L; ++i) {
        e = csa::launch_sort_rows(out_idx[i], score_dst[i], (long long)probs[0]->B * probs[0]->S_q, cap, st);
        if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "sort launch failed: %s", hipGetErrorString(e));
      }
    }
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_project(const void* x, const void* w, int64_t M, int32_t N, int32_t K, int32_t out_dtype, void* y,
                       void* hip_stream) {
  try {
    if (M < 0) return fail(CSA_ERR_INVALID, "M=%lld must be >= 0", (long long)M);
    if (N < 1 || K < 1) return fail(CSA_ERR_INVALID, "N=%d and K=%d must be >= 1", N, K);
    if (out_dtype != CSA_BF16 && out_dtype != CSA_F32) return fail(CSA_ERR_INVALID, "out_dtype must be CSA_BF16 or CSA_F32");
    if (K % csa::PJ_BK) return fail(CSA_ERR_UNSUPPORTED, "K=%d must be a multiple of %d", K, csa::PJ_BK);
    if (N > CSA_MAX_PROJECT_N) return fail(CSA_ERR_UNSUPPORTED, "N=%d above %d", N, CSA_MAX_PROJECT_N);
    if (M > csa::project_rows_limit())
      return fail(CSA_ERR_UNSUPPORTED, "M=%lld above %lld rows per call", (long long)M, csa::project_rows_limit());
    if (M == 0) return ok();
    if (!x || !w || !y) return fail(CSA_ERR_INVALID, "x, w and y must not be NULL");
    if ((uintptr_t)x % 16 || (uintptr_t)w % 16) return fail(CSA_ERR_INVALID, "x and w must be 16-byte aligned");
    if ((uintptr_t)y % (out_dtype == CSA_F32 ? 4 : 2)) return fail(CSA_ERR_INVALID, "y is misaligned");
    csa::ProjArgs a{x, w, y, (long long)M, N, K, out_dtype == CSA_F32 ? 1 : 0};
    const hipError_t e = csa::launch_project(a, N >= 256 ? 0 : 1, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "projection launch failed: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_index_topk_interleaved(const csa_problem* prob, int32_t P, int32_t k_local, uint32_t flags,
                                      int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                      void* hip_stream) {
  try {
    csa_status s = validate_problem(prob);
    if (s != CSA_OK) return s;
    if ((s = validate_flags(flags)) != CSA_OK) return s;
    if ((s = validate_k(k_local, "k_local")) != CSA_OK) return s;
    if (P < 1) return fail(CSA_ERR_INVALID, "P=%d < 1", P);
    if ((long long)P * k_local > (1ll << 30)) return fail(CSA_ERR_UNSUPPORTED, "P*k_local too large");
    if (!out_idx) return fail(CSA_ERR_INVALID, "out_idx is NULL");
    return run_prefill_family(prob, csa::MODE_INTERLEAVED, k_local, P, flags, 0ull, out_idx, out_score, nullptr,
                              ws, ws_bytes, hip_stream);
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

}  // extern "C"

namespace {

struct AttnPlan {
  int nsplit;
  size_t opart_bytes, stat_bytes, total;
};

// Workgroups per query row: about 256 workgroups in all (one per CU), never
// more than the row has AT_CHUNK-entry chunks.
AttnPlan plan_attention(const csa_attn_problem* p, int n_sel) {
  AttnPlan pl;
  const long long rows = (long long)p->B * p->S_q;
  const int nchunk = (n_sel + csa::AT_CHUNK - 1) / csa::AT_CHUNK;
  long long ns = (256 + rows - 1) / rows;
  ns = std::max(1ll, std::min(ns, (long long)nchunk));
  pl.nsplit = (int)ns;
  pl.opart_bytes = align_up((size_t)rows * pl.nsplit * csa::AT_H * csa::AT_D * sizeof(float));
  pl.stat_bytes = align_up((size_t)rows * pl.nsplit * csa::AT_H * sizeof(float));
  pl.total = pl.opart_bytes + 2 * pl.stat_bytes;
  return pl;
}

csa_status validate_attention(const csa_attn_problem* p, int n_sel) {
  if (!p) return fail(CSA_ERR_INVALID, "problem is NULL");
  if (p->struct_size != sizeof(csa_attn_problem)) return fail(CSA_ERR_INVALID, "struct_size mismatch");
  if (p->B < 1 || p->S_q < 1 || p->T < 1) return fail(CSA_ERR_INVALID, "B, S_q and T must be >= 1");
  if (n_sel < 1) return fail(CSA_ERR_INVALID, "n_sel=%d < 1", n_sel);
  if (p->H != csa::AT_H || p->Dk != csa::AT_D || p->Dv != csa::AT_D)
    return fail(CSA_ERR_UNSUPPORTED, "sparse attention needs H=64, Dk=Dv=128 (got H=%d Dk=%d Dv=%d)", p->H, p->Dk, p->Dv);
  if (!p->q || !p->k || !p->v) return fail(CSA_ERR_INVALID, "q, k and v must not be NULL");
  if ((long long)p->B * p->S_q > (1ll << 31) - 1) return fail(CSA_ERR_UNSUPPORTED, "too many query rows");
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_attention_workspace_size(const csa_attn_problem* prob, int32_t n_sel, size_t* bytes) {
  try {
    if (!bytes) return fail(CSA_ERR_INVALID, "bytes is NULL");
    const csa_status s = validate_attention(prob, n_sel);
    if (s != CSA_OK) return s;
    *bytes = plan_attention(prob, n_sel).total;
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_sparse_attention(const csa_attn_problem* prob, const int32_t* idx, int32_t n_sel, float scale,
                                float* out, void* ws, size_t ws_bytes, void* hip_stream) {
  try {
    const csa_status s = validate_attention(prob, n_sel);
    if (s != CSA_OK) return s;
    if (!idx || !out) return fail(CSA_ERR_INVALID, "idx and out must not be NULL");
    if (!std::isfinite(scale)) return fail(CSA_ERR_INVALID, "scale must be finite");
    const AttnPlan pl = plan_attention(prob, n_sel);
    if (ws_bytes < pl.total || !ws) return fail(CSA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, pl.total);
    if ((uintptr_t)ws % 16) return fail(CSA_ERR_INVALID, "workspace must be 16-byte aligned");
    csa::AttnArgs a{};
    a.q = prob->q; a.k = prob->k; a.v = prob->v; a.idx = idx;
    a.B = prob->B; a.S_q = prob->S_q; a.T = prob->T; a.n_sel = n_sel; a.scale = scale;
    a.nsplit = pl.nsplit;
    char* wp = (char*)ws;
    a.opart = (float*)wp;
    a.mpart = (float*)(wp + pl.opart_bytes);
    a.lpart = (float*)(wp + pl.opart_bytes + pl.stat_bytes);
    a.out = out;
    hipError_t e = csa::launch_attention(a, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "attention launch failed: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_union_rows(const int32_t* const* lists, const int32_t* widths, int32_t L, int64_t rows, int32_t T,
                          int32_t cap, int32_t* out_idx, int32_t* out_count, void* hip_stream) {
  try {
    static_assert(CSA_MAX_UNION_LISTS == csa::UN_MAX_LISTS && CSA_MAX_UNION_T == csa::UN_MAX_T, "union limits");
    if (L < 1 || L > CSA_MAX_UNION_LISTS) return fail(CSA_ERR_INVALID, "L=%d outside [1, %d]", L, CSA_MAX_UNION_LISTS);
    if (!lists || !widths) return fail(CSA_ERR_INVALID, "lists and widths must not be NULL");
    if (rows < 0) return fail(CSA_ERR_INVALID, "rows=%lld < 0", (long long)rows);
    if (T < 1 || cap < 1) return fail(CSA_ERR_INVALID, "T and cap must be >= 1");
    if (T > CSA_MAX_UNION_T) return fail(CSA_ERR_UNSUPPORTED, "T=%d > %d", T, CSA_MAX_UNION_T);
    if (rows > max_rows_per_dispatch(csa::UN_THREADS)) return fail(CSA_ERR_UNSUPPORTED, "too many rows");
    csa::UnionArgs a{};
    for (int i = 0; i < L; ++i) {
      if (widths[i] < 1) return fail(CSA_ERR_INVALID, "widths[%d]=%d < 1", i, widths[i]);
      if (rows > 0 && !lists[i]) return fail(CSA_ERR_INVALID, "lists[%d] is NULL", i);
      a.list[i] = lists[i];
      a.width[i] = widths[i];
    }
    if (rows > 0 && !out_idx) return fail(CSA_ERR_INVALID, "out_idx must not be NULL");
    a.L = L; a.T = T; a.cap = cap; a.out_idx = out_idx; a.out_count = out_count;
    hipError_t e = csa::launch_union(a, rows, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "union launch failed: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

csa_status csa_set_recall(const int32_t* sel, int32_t n_sel, const int32_t* ref, int32_t n_ref, int64_t rows,
                          int32_t T, float* out_recall, void* ws, size_t ws_bytes, void* hip_stream) {
  (void)ws;
  (void)ws_bytes;
  try {
    if (rows < 0) return fail(CSA_ERR_INVALID, "rows=%lld < 0", (long long)rows);
    if (n_sel < 1 || n_ref < 1 || T < 1) return fail(CSA_ERR_INVALID, "n_sel, n_ref and T must be >= 1");
    if (n_ref > 8192) return fail(CSA_ERR_UNSUPPORTED, "n_ref=%d > 8192", n_ref);
    if (rows > 0 && (!sel || !ref || !out_recall)) return fail(CSA_ERR_INVALID, "sel, ref and out_recall must not be NULL");
    if (rows > max_rows_per_dispatch(256)) return fail(CSA_ERR_UNSUPPORTED, "too many rows");
    hipError_t e = csa::launch_recall(sel, n_sel, ref, n_ref, rows, T, out_recall, (hipStream_t)hip_stream);
    if (e != hipSuccess) return fail(CSA_ERR_DEVICE, "recall launch failed: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(CSA_ERR_INVALID, "internal error");
  }
}

}  // extern "C"
