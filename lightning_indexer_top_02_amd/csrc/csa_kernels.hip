// HIP kernels (gfx950) for the CSA lightning-indexer top-k step.
//
// Score (per query t, key s):  I = sum_j w[t,j] * max(q[t,j] . k[s], 0).
// Every kernel streams key tiles, forms scores in registers and feeds a
// per-query running top-k; the [B,S,H,T] score tensor is never formed.
//
// Prefill family (top-k, threshold, interleaved partitions):
//   persistent grid; a workgroup owns consecutive query rows, one per wave
//   (8 in the MFMA kernel, 4 in the generic one).  Per step the wave produces
//   64 (query, key) scores, one per lane, filters them against the query's
//   running threshold key and appends
//   survivors to the query's candidate buffer in the workspace.  A full
//   buffer is compacted to the exact top-k (which raises the threshold); at
//   the end the exact top-k of the buffer is emitted.
// Decode: scores of a few queries against a long key range, split across
//   many workgroups (HBM-bound), then one workgroup per row selects.
#include <mutex>

#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

// ============================================================ shared pieces

// max(x, 0) as one integer max on the bits: negative floats (and -0.0) are
// negative as int32, non-negative ones keep their order; -0.0 becomes +0.0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Two column tiles' per-lane partial sums (each lane holds half of its key's
// heads; lane l and lane l^32 hold the two halves): returns, in lanes 0-31,
// the full score of tile 0's key (l & 31) and, in lanes 32-63, tile 1's.
// v_permlane32_swap moves tile 0's upper half down and tile 1's lower half up.
__device__ __forceinline__ float half_swap_sum(float p0, float p1) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int row_visible(const PrefillArgs& a, int b, int row, int part) {
  if (row >= a.S_q) return 0;
  long long v = a.causal ? (a.q_pos0 + row) / a.m + 1 : (long long)a.T;
  if (v > a.T) v = a.T;
  if (a.kv_len) {
    long long kv = a.kv_len[b];
    if (kv < 0) kv = 0;
    if (v > kv) v = kv;
  }
  if (a.P > 1) v = v > part ? (v - part + a.P - 1) / a.P : 0;   // keys p, p+P, ... below v
  return (int)v;
}

// Top-k state of the wave's query row (wave-uniform except lo/hi).  The
// append threshold is kept as a (score, index) pair: a key (s, i) may enter
// iff s > thr_s, or s == thr_s and i <= thr_i -- the same total order as the
// 64-bit keys, with float compares (-0.0 == +0.0).
struct Slot {
  u64* cand;     // candidate buffer (C keys)
  int cnt;       // keys in it
  float thr_s;   // append threshold (inclusive on the index)
  uint32_t thr_i;
  int surv;      // threshold mode: keys >= thr_fixed seen
  float lo, hi;  // per lane: bounds on the scores this lane appended
};

// Candidate buffers and output rows are written once and read at most once
// more: their loads and stores are non-temporal, so that they stream past L2
// instead of evicting the key tiles every workgroup re-reads there.  (Dense
// score rows, read back right after by the select kernel, stay cacheable:
// measured faster.)

// Inclusive key bound X (keys >= X pass) as a (score, index) threshold.
__device__ __forceinline__ void key_to_thr(u64 X, float& ts, uint32_t& ti) {
  if (X == 0ull) {                                    // everything passes
    ts = -__builtin_inff();
    ti = 0xFFFFFFFFu;
  } else {
    ts = key_score(X);
    ti = 0xFFFFFFFFu - (uint32_t)X;
  }
}

__device__ __forceinline__ bool passes(float s, uint32_t i, float ts, uint32_t ti) {
  return s > ts || (s == ts && i <= ti);
}

// Exact top-kk of buf[0..n) (n > kk) in two streaming passes: a linear-bin
// histogram between the lanes' score bounds lo / hi, then one pass that hands
// every key of a bin above the bin holding rank kk to put(key, position)
// (positions 0, 1, ... in buffer order) and gathers that bin's keys into the
// LDS list, whose exact rank-r key T is found there; the list's keys >= T
// follow (positions up to kk - 1).  Returns T, or 0 when the bins cannot
// narrow the rank (no usable range, or a bin too crowded for the list): the
// caller then takes the general selection and nothing has been put.  put
// may write back into buf: a key goes to a position at or below the one it
// was read from.
template <typename Put>
__device__ __forceinline__ u64 wave_binned_select(const u64* buf, int n, int kk, uint32_t* hist, u64* list,
                                                  float lo, float hi, Put put) {
  const int l = lane_id();
  LinBins lb;
  if (!lin_bins_ok(lo, hi, lb)) return 0ull;
  wave_clear_hist(hist, SEL_BINS);
  wave_lds_sync();
  wave_stream(buf, n, [&](u64 v, int) {
    if (v) atomicAdd(&hist[lb(v)], 1u);
  });
  wave_lds_sync();
  const BinPick pk = wave_pick_bin(hist, SEL_BINS, kk);
  wave_lds_sync();
  const int r = kk - pk.above;
  if (pk.count <= 0 || pk.count > WAVE_LIST || pk.count < r) return 0ull;
  int w = 0, wl = 0;
  wave_stream(buf, n, [&](u64 v, int) {               // 0 = past the end (no key is 0)
    const int b = v ? lb(v) : -1;
    const bool up = b > pk.bin, at = b == pk.bin;
    const u64 mu = ballot(up), ma = ballot(at);
    if (up) put(v, w + lanes_below(mu));
    if (at) list[wl + lanes_below(ma)] = v;
    w += __popcll(mu);
    wl += __popcll(ma);
  });
  wave_lds_sync();
  const u64 T = wave_list_kth(list, wl, kk - w, hist);
  wave_lds_sync();
  for (int i0 = 0; i0 < wl; i0 += WAVE) {              // the rank bin's keys >= T
    const int i = i0 + l;
    const u64 v = i < wl ? list[i] : 0ull;
    const bool keep = i < wl && v >= T;
    const u64 m = ballot(keep);
    if (keep) put(v, w + lanes_below(m));
    w += __popcll(m);
  }
  wave_lds_sync();
  return T;
}

// Keep the exact top-kk of buf[0..cnt) in place (cnt > kk); returns the kk-th
// key.  Streams the buffer: the wave's MFMA operands stay in registers meanwhile.
__device__ __forceinline__ u64 wave_compact(u64* buf, int cnt, int kk, uint32_t* hist, u64* list, float lo,
                                           float hi) {
  wave_own_stores_visible();
  lo = wave_min_f32(lo);
  hi = wave_max_f32(hi);
  const u64 Tb = wave_binned_select(buf, cnt, kk, hist, list, lo, hi,
                                    [&](u64 v, int pos) { __builtin_nontemporal_store(v, &buf[pos]); });
  if (Tb) return Tb;
  const u64 T = wave_select_kth_stream(buf, cnt, kk, hist, list, lo, hi);
  int w = 0;
  wave_stream(buf, cnt, [&](u64 v, int) {        // in order; writes never pass the reads
    const bool keep = v >= T && v != 0ull;
    const u64 m = ballot(keep);
    if (keep) __builtin_nontemporal_store(v, &buf[w + lanes_below(m)]);
    w += __popcll(m);
  });
  return T;
}

// Offer one (score, index) per lane (valid lanes only) to the wave's query.
template <int MODE>
__device__ __forceinline__ void wave_offer(Slot& st, float score, uint32_t idx, bool valid, const PrefillArgs& a,
                                           uint32_t* hist, u64* list) {
  if (st.cnt + WAVE > a.C) {                          // make room: at most 64 appends per offer
    const u64 T = wave_compact(st.cand, st.cnt, a.kk, hist, list, st.lo, st.hi);
    st.cnt = a.kk;
    st.lo = key_score(T);                              // every survivor scores >= the kk-th
    // new keys must beat the kk-th key T (and, in threshold mode, still pass thr_fixed)
    const u64 X = (MODE == MODE_THRESHOLD && a.thr_fixed > T + 1ull) ? a.thr_fixed : T + 1ull;
    key_to_thr(X, st.thr_s, st.thr_i);
  }
  if (MODE == MODE_THRESHOLD) {
    float fs;
    uint32_t fi;
    key_to_thr(a.thr_fixed, fs, fi);
    st.surv += __popcll(ballot(valid && passes(score, idx, fs, fi)));
  }
  const bool keep = valid && passes(score, idx, st.thr_s, st.thr_i);
  const u64 m = ballot(keep);
  if (keep) {
    __builtin_nontemporal_store(make_key(score, idx), &st.cand[st.cnt + lanes_below(m)]);
    st.lo = fminf(st.lo, score);
    st.hi = fmaxf(st.hi, score);
  }
  st.cnt += __popcll(m);
}

__device__ __forceinline__ void emit_key(u64 x, int pos, int kk, int32_t* oi, float* os) {
  if (pos < kk) {                                     // exactly kk pass; the bound only guards the row
    __builtin_nontemporal_store(key_index(x), &oi[pos]);
    if (os) __builtin_nontemporal_store(key_score(x), &os[pos]);
  }
}

// Candidate buffers up to this size are selected from registers: one load
// pass with every load in flight instead of two latency-bound streaming
// passes.
constexpr int EMIT_REGS = 66;

// Emit the exact top-kk of the n_keys nonzero keys key(j) (all of them when
// n_keys <= kk; key(j) is the key of element j*WAVE + lane for j*WAVE < n, 0
// = empty) to one output row, in no particular order; returns the number
// written.  lo/hi: per-lane score bounds of the nonzero keys.  One histogram
// pass over linear score bins finds the bin holding rank kk; one more pass
// emits every key of a higher bin and gathers the bin's own keys into `list`,
// whose top r are resolved exactly and emitted last.  Keys are recomputed by
// key(j) on each pass, so callers may hold them in a compact form.
template <int R, typename KeyAt>
__device__ __forceinline__ int wave_emit_keys_at(KeyAt key, int n, int n_keys, int kk, uint32_t* hist, u64* list,
                                                 float lo, float hi, int32_t* oi, float* os) {
  const int l = lane_id();
  int w = 0;
  auto emit_ge = [&](u64 T) {                          // every key >= T (T >= 1 skips empty slots)
    key.fresh();
    const int nn = fresh_bound(n);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j * WAVE < nn) {
        const u64 v = key(j);
        const bool keep = v >= T;
        const u64 m = ballot(keep);
        if (keep) emit_key(v, w + lanes_below(m), kk, oi, os);
        w += __popcll(m);
      }
      __builtin_amdgcn_sched_barrier(0);               // one slot at a time: short mask live ranges
    }
    return w < kk ? w : kk;
  };
  if (n_keys <= kk) return emit_ge(1ull);
  lo = wave_min_f32(lo);
  hi = wave_max_f32(hi);
  LinBins lb;
  if (!lin_bins_ok(lo, hi, lb)) return emit_ge(wave_radix_kth_at<R>(key, n, kk, hist, AnyKey{}));
  wave_clear_hist(hist, SEL_BINS);
  wave_lds_sync();
  key.fresh();
  int nn = fresh_bound(n);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * WAVE < nn) {
      const u64 v = key(j);
      if (v) atomicAdd(&hist[lb(v)], 1u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wave_lds_sync();
  const BinPick pk = wave_pick_bin(hist, SEL_BINS, kk);
  wave_lds_sync();
  const int r = kk - pk.above;
  if (pk.count > WAVE_LIST || pk.count < r)           // crowded bin (or inconsistent counts): exact radix
    return emit_ge(wave_radix_kth_at<R>(key, n, r, hist, InBin{lb, pk.bin}));
  int lc = 0;
  key.fresh();
  nn = fresh_bound(n);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * WAVE < nn) {
      const u64 v = key(j);
      const int bin = v ? lb(v) : -1;
      const bool up = bin > pk.bin, at = bin == pk.bin;
      const u64 mu = ballot(up), ma = ballot(at);
      if (up) emit_key(v, w + lanes_below(mu), kk, oi, os);
      if (at) list[lc + lanes_below(ma)] = v;
      w += __popcll(mu);
      lc += __popcll(ma);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  wave_lds_sync();
  // the boundary bin: its top r keys (lc >= r keys, all distinct)
  const u64 T = r == lc ? 1ull : wave_list_kth(list, lc, r, hist);
  for (int base = 0; base < lc; base += WAVE) {
    const int i = base + l;
    const u64 v = i < lc ? list[i] : 0ull;
    const bool keep = i < lc && v >= T;
    const u64 m = ballot(keep);
    if (keep) emit_key(v, w + lanes_below(m), kk, oi, os);
    w += __popcll(m);
  }
  wave_lds_sync();
  return w < kk ? w : kk;
}

template <int R>
__device__ __forceinline__ int wave_emit_keys_regs(const u64 (&x)[R], int n, int n_keys, int kk, uint32_t* hist,
                                                   u64* list, float lo, float hi, int32_t* oi, float* os) {
  return wave_emit_keys_at<R>(ArrayKeys<R>{x}, n, n_keys, kk, hist, list, lo, hi, oi, os);
}

__device__ __forceinline__ int wave_emit_cand_stream(const Slot& st, int kk, uint32_t* hist, u64* list, int32_t* oi,
                                                     float* os);

// Emit the exact top-kk of the candidate list buf[0..cnt) (all of it when
// cnt <= kk); returns the number written.
__device__ __forceinline__ int wave_emit_cand(const Slot& st, int kk, uint32_t* hist, u64* list, int32_t* oi,
                                              float* os) {
  const int l = lane_id();
  wave_own_stores_visible();
  if (st.cnt <= EMIT_REGS * WAVE) {
    u64 x[EMIT_REGS];
#pragma unroll
    for (int j = 0; j < EMIT_REGS; ++j) {
      const int i = j * WAVE + l;
      x[j] = __builtin_nontemporal_load(&st.cand[i < st.cnt ? i : (st.cnt > 0 ? st.cnt - 1 : 0)]);
    }
#pragma unroll
    for (int j = 0; j < EMIT_REGS; ++j)                 // (unconditional loads above: all in flight)
      if (j * WAVE + l >= st.cnt) x[j] = 0ull;
    return wave_emit_keys_regs(x, st.cnt, st.cnt, kk, hist, list, st.lo, st.hi, oi, os);
  }
  return wave_emit_cand_stream(st, kk, hist, list, oi, os);
}

// The same by streaming the buffer (any length; registers stay free).
__device__ __forceinline__ int wave_emit_cand_stream(const Slot& st, int kk, uint32_t* hist, u64* list, int32_t* oi,
                                                     float* os) {
  if (st.cnt > kk) {                                  // two passes when the bins narrow the rank
    const float lo = wave_min_f32(st.lo), hi = wave_max_f32(st.hi);
    if (wave_binned_select(st.cand, st.cnt, kk, hist, list, lo, hi,
                           [&](u64 v, int pos) { emit_key(v, pos, kk, oi, os); }))
      return kk;
  }
  const u64 T = st.cnt > kk ? wave_select_kth_stream(st.cand, st.cnt, kk, hist, list, st.lo, st.hi) : 1ull;
  int w = 0;
  wave_stream(st.cand, st.cnt, [&](u64 v, int) {
    const bool keep = v >= T;                          // T >= 1 excludes slots past the end
    const u64 m = ballot(keep);
    if (keep) emit_key(v, w + lanes_below(m), kk, oi, os);
    w += __popcll(m);
  });
  return w < kk ? w : kk;
}

// Pad an output row after its first w entries with -1 / -inf.
__device__ __forceinline__ void wave_pad_row(int w, int kk, int32_t* oi, float* os) {
  for (int i = w + lane_id(); i < kk; i += WAVE) {
    oi[i] = -1;
    if (os) os[i] = -__builtin_inff();
  }
}

__device__ __forceinline__ void decode_item(const PrefillArgs& a, int it, int& b, int& qb, int& part) {
  part = it % a.P;
  b = (it / a.P) % a.B;
  qb = a.nqb - 1 - it / (a.P * a.B);                  // heaviest (latest) query blocks first
}

// Item processed by this workgroup in round r (snake order over the grid).
__device__ __forceinline__ int round_item(int r) {
  const int G = gridDim.x;
  return r * G + ((r & 1) ? (G - 1 - (int)blockIdx.x) : (int)blockIdx.x);
}

// Does any row of the block need scores (more visible keys than kk, scores
// requested, or threshold mode)?  Also the block's largest visible count.
template <int MODE, int ROWS = PF_ROWS>
__device__ __forceinline__ bool block_needs_scores(const PrefillArgs& a, int b, int qb, int part, int& vis_max) {
  vis_max = 0;
  bool need = MODE == MODE_THRESHOLD || a.need_scores;
  for (int r = 0; r < ROWS; ++r) {
    const int v = row_visible(a, b, qb * ROWS + r, part);
    vis_max = v > vis_max ? v : vis_max;
    need = need || v > a.kk;
  }
  return need;
}

__device__ __forceinline__ int32_t* out_row(const PrefillArgs& a, int b, int row, int part) {
  return a.out_idx + ((size_t)b * a.S_q + row) * a.out_stride + (size_t)part * a.kk;
}

// A row whose visible keys all fit (vis <= kk) and whose scores are not asked
// for: the selection is every visible key.
__device__ __forceinline__ void wave_emit_all_visible(const PrefillArgs& a, int b, int row, int part, int vis) {
  const int l = lane_id();
  int32_t* oi = out_row(a, b, row, part);
  for (int i = l; i < a.kk; i += WAVE) __builtin_nontemporal_store(i < vis ? part + a.P * i : -1, &oi[i]);
}

template <int MODE>
__device__ __forceinline__ void finish_row(const PrefillArgs& a, Slot& st, int b, int row, int part, uint32_t* hist, u64* list) {
  if (row >= a.S_q) return;
  const size_t orow = (size_t)b * a.S_q + row;
  float* os = a.out_score ? a.out_score + orow * a.out_stride + (size_t)part * a.kk : nullptr;
  int32_t* oi = out_row(a, b, row, part);
  wave_pad_row(wave_emit_cand(st, a.kk, hist, list, oi, os), a.kk, oi, os);
  if (MODE == MODE_THRESHOLD && lane_id() == 0) a.out_count[orow] = st.surv;
}

__device__ __forceinline__ void slot_init(Slot& st, u64* cand, const PrefillArgs& a, int mode) {
  st.cand = cand;
  st.cnt = 0;
  key_to_thr(mode == MODE_THRESHOLD ? a.thr_fixed : 0ull, st.thr_s, st.thr_i);
  st.surv = 0;
  st.lo = __builtin_inff();
  st.hi = -__builtin_inff();
}

// ============================================================ LDS staging helpers

// s_waitcnt vmcnt(n) with no wait on the other counters (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 l
// (lds is the same in every lane).  Written as asm so that the compiler does
// not treat every later LDS access as a possible reader of the in-flight load
// (it would drain vmcnt to 0 before each one); the caller orders the data
// with explicit vmcnt waits instead.  The instruction has no register results
// (only its address operand, read at issue), and the kernel using it holds
// nothing else in M0 (only these sequences write it), so clobbering M0 here
// is safe.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);   // wave-uniform LDS base
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (the instruction's saddr form): the per-step address update is
// scalar work only.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m)
               : "memory", "m0");
}

// ============================================================ MFMA prefill
//
// bf16, H = 64 heads, D = 128.  A wave holds its query's 64 heads x 128 as
// MFMA A operands (2 row tiles of 32 heads, 64 VGPRs) and its 64 head weights
// in registers, and per step multiplies them with two 32-key column tiles read
// from LDS: v_mfma_f32_32x32x16_bf16, fp32 accumulation, 8 k-steps over D.
// Output lane l holds key column (l & 31) and 16 heads of a row tile; ReLU and
// the head weights are applied in registers; exchanging the two column tiles'
// half-wave partial sums leaves lanes 0-31 with the scores of tile 0 and lanes
// 32-63 with those of tile 1.  Each wave filters its row's scores into a
// candidate list (compacted to the top-kk when full) and selects the row's
// final top-kk from it at the end of the query block.

constexpr int MH = 64, MD = 128;
// A key tile (PF_KTILE keys x 256 B) sits in LDS as groups of 16 keys; inside
// a group the 16-byte d-chunks are plane-major:
//     byte(key, chunk) = (key / 16) * 4096 + chunk * 256 + (key % 16) * 16.
// A wave's direct-to-LDS load (global_load_lds_dwordx4) fills 1 KB contiguous
// = 16 keys x 4 chunks (64 B of each key row), and the MFMA B-operand read
// (32 keys x one chunk per half-wave) hits 16 distinct bank quads per 16
// lanes, with the k-step in the instruction's immediate offset.
constexpr int KT_BYTES = PF_KTILE * MD * 2;

// ============================================================ MFMA prefill, ping-pong
//
// The computation above with eight waves (one query row each) per workgroup
// and one workgroup per CU, so every SIMD runs two waves of one workgroup:
// wave w and wave w + 4.  A SIMD overlaps one wave's MFMAs with another
// wave's VALU work, but not with its own, and waves that run the same phase
// at the same time only compete.  So the two groups of four waves run half a
// step apart: each step of a wave is an MFMA half (B operands from LDS, 32
// MFMAs) and a VALU half (ReLU, head weights, offer, key-tile requests), and
// workgroup barriers between the halves keep group 1's MFMA half under group
// 0's VALU half and the other way round.  Each key tile in LDS serves eight
// rows.  A ring of PF2_NSTAGE = 4 tiles: the tile three steps ahead is
// requested in a VALU half, after every reader of the stage it overwrites
// (step t - 1, both groups) has passed a barrier, and each wave waits for its
// own requests of tile t + 1 at the end of its MFMA half t, before the
// barrier after which either group reads that tile.  The VALU half is kept
// short, since it is the longer of the two: scores become 64-bit keys at
// once and the running threshold is a key, the candidate stores and the
// key-tile requests take wave-uniform bases in SGPRs with 32-bit lane
// offsets.  The arithmetic and its order are those of the other kernels
// (bitwise the same scores).
// Running top-k state of one wave's query row in the MFMA kernel, kept in
// key form: a key (order bits of the score, ~index) may enter iff key >= X,
// the same total order as Slot's (score, index) threshold.  lo_o / hi_o (per
// lane) are the order bits of the smallest and largest score this lane
// appended (unsigned min / max of order bits = min / max of the scores).
struct KeySlot {
  u64* cand;
  int cnt;
  u64 X;
  int surv;
  uint32_t lo_o, hi_o;
};

// The compaction of a full candidate buffer, out of line: it runs a few
// times per query row, and inlined its scalar temporaries would crowd the
// MFMA kernel's tile loop into spilling SGPRs.
__device__ __attribute__((noinline)) u64 wave_compact_call(u64* buf, int cnt, int kk, uint32_t* hist, u64* list,
                                                           float lo, float hi) {
  return wave_compact(buf, cnt, kk, hist, list, lo, hi);
}

// Offer one key per lane (valid lanes only) to the wave's query row.
template <int MODE>
__device__ __forceinline__ void key_offer(KeySlot& st, u64 key, bool valid, const PrefillArgs& a, uint32_t* hist,
                                          u64* list) {
  if (st.cnt + WAVE > a.C) {                          // make room: at most 64 appends per offer
    const u64 T = wave_compact_call(st.cand, st.cnt, a.kk, hist, list, order_bits_score(st.lo_o),
                                    order_bits_score(st.hi_o));
    st.cnt = a.kk;
    st.lo_o = (uint32_t)(T >> 32);                    // every survivor scores >= the kk-th
    st.X = (MODE == MODE_THRESHOLD && a.thr_fixed > T + 1ull) ? a.thr_fixed : T + 1ull;
  }
  if (MODE == MODE_THRESHOLD) st.surv += __popcll(ballot(valid && key >= a.thr_fixed));
  const bool keep = valid && key >= st.X;
  const u64 m = ballot(keep);
  if (keep) {
    const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)st.cnt));
    __builtin_nontemporal_store(key, (u64*)((char*)st.cand + pos * 8u));
    const uint32_t o = (uint32_t)(key >> 32);
    st.lo_o = o < st.lo_o ? o : st.lo_o;
    st.hi_o = o > st.hi_o ? o : st.hi_o;
  }
  st.cnt += __popcll(m);
}

// Order bits of a score that is never -0.0 (see the kernel): no -0.0 fold.
__device__ __forceinline__ uint32_t order_bits_nz(float s) {
  const uint32_t u = __float_as_uint(s);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

template <int MODE>
__global__ __launch_bounds__(PF2_THREADS, 1) void prefill_mfma2_kernel(PrefillArgs a) {
  constexpr int NW = PF2_THREADS / WAVE;           // 8 waves
  constexpr int NB = 16 / NW;                       // 1 KB tile blocks requested per wave
  static_assert((PF2_NSTAGE & (PF2_NSTAGE - 1)) == 0 && PF2_NSTAGE >= 4, "ring of 2^n >= 4 stages");
  __shared__ __attribute__((aligned(1024))) char ktile[PF2_NSTAGE][KT_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[NW][SEL_BINS];
  __shared__ u64 list_all[NW][WAVE_LIST];

  const int tid = threadIdx.x, l = tid & (WAVE - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid / WAVE);   // wave-uniform: scalar address math
  const int grp = wv / 4;                           // group 0: waves 0-3, group 1: waves 4-7
  uint32_t* hist = hist_all[wv];
  u64* list = list_all[wv];
  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const int b_off = ((l >> 4) & 1) * 4096 + (l >> 5) * 256 + (l & 15) * 16;
  uint32_t doff[NB], dlds[NB];
#pragma unroll
  for (int e = 0; e < NB; ++e) {
    const int blk = e * NW + wv, row = (blk >> 2) * 16 + (l & 15), chunk = (blk & 3) * 4 + (l >> 4);
    doff[e] = (uint32_t)(((size_t)row * a.P * MD + chunk * 8) * 2);
    dlds[e] = lds_addr(&ktile[0][blk * 1024]);
  }
  const uint32_t tile_step = (uint32_t)a.P * PF_KTILE;        // key rows per tile
  const size_t tile_bytes = (size_t)tile_step * MD * 2;

  for (int r = 0;; ++r) {
    const int it = round_item(r);
    if (r * (int)gridDim.x >= a.n_items) break;
    if (it >= a.n_items) continue;
    int b, qb, part;
    decode_item(a, it, b, qb, part);
    int vis_max;
    const bool need = block_needs_scores<MODE, PF2_ROWS>(a, b, qb, part, vis_max);   // uniform
    const int row = qb * PF2_ROWS + wv;               // this wave's query row
    const int vis = row_visible(a, b, row, part);
    if (!need) {
      if (row < a.S_q) wave_emit_all_visible(a, b, row, part, vis);
      continue;
    }

    bf16x8 A[2][8];
    float wl[2][16];
    const int rq = row < a.S_q ? row : a.S_q - 1;     // rows past the end compute on a valid row, emit nothing
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const bf16x8* src = (const bf16x8*)(Q + (((size_t)b * a.S_q + rq) * MH + rt * 32 + (l & 31)) * MD);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) A[rt][kk] = src[2 * kk + (l >> 5)];
      const float* wrow = a.w + ((size_t)b * a.S_q + rq) * MH + rt * 32 + 4 * (l >> 5);
#pragma unroll
      for (int i = 0; i < 16; ++i) wl[rt][i] = wrow[8 * (i >> 2) + (i & 3)];
    }
    KeySlot st;
    st.cand = a.cand + ((size_t)blockIdx.x * PF2_ROWS + wv) * a.C;
    st.cnt = 0;
    st.X = MODE == MODE_THRESHOLD ? a.thr_fixed : 0ull;
    st.surv = 0;
    st.lo_o = 0xFF800000u;                            // order bits of +inf
    st.hi_o = 0x007FFFFFu;                            // order bits of -inf
    // ~index of this lane's key in step t: nidx0 - t * tile_step
    const uint32_t nidx0 = 0xFFFFFFFFu - (uint32_t)(part + a.P * l);

    const int ntiles = (vis_max + PF_KTILE - 1) / PF_KTILE;
    const size_t kseq = (size_t)b * a.T;
    const char* kbase = (const char*)(K + (kseq + (size_t)part) * MD);
    // tiles 0 .. nfull-1 hold PF_KTILE keys below T: part + P (64 t + 63) < T
    const long long lim = (long long)a.T - 1 - part - (long long)(PF_KTILE - 1) * a.P;
    const int nfull = lim < 0 ? 0 : (int)(lim / tile_step + 1 < ntiles ? lim / tile_step + 1 : ntiles);
    // this wave's share of tile t (blocks wv and wv + 8, 1 KB each) into stage buf
    auto load_tile = [&](int t, int buf, const char* base) {
      if (t < nfull) {
#pragma unroll
        for (int e = 0; e < NB; ++e) dma16s(base, doff[e], dlds[e] + (uint32_t)buf * KT_BYTES);
      } else {
#pragma unroll
        for (int e = 0; e < NB; ++e) {
          const int blk = e * NW + wv, gk = blk >> 2, quad = blk & 3;
          int j = t * PF_KTILE + gk * 16 + (l & 15);
          j = j < vis_max ? j : vis_max - 1;          // rows past the end: any valid row (masked later)
          const int chunk = quad * 4 + (l >> 4);
          dma16(K + (kseq + (size_t)part + (size_t)a.P * j) * MD + chunk * 8, dlds[e] + (uint32_t)buf * KT_BYTES);
        }
      }
    };
    __syncthreads();                                  // previous item's readers are done with the stages
    const int t_part = grp == 0 ? ntiles - 2 : -1;    // steps whose MFMA half ends with a partial wait
    const char* knext = kbase;                        // global address of the next tile to request
#pragma unroll
    for (int s0 = 0; s0 < PF2_NSTAGE - 1; ++s0) {
      if (s0 < ntiles) load_tile(s0, s0, knext);
      knext += tile_bytes;
    }
    wait_vmcnt<0>();
    __syncthreads();
    // first B operands of step 0 (each MFMA half starts with its first B operands in registers)
    bf16x8 b0 = *(const bf16x8*)(&ktile[0][b_off]);
    bf16x8 b1 = *(const bf16x8*)(&ktile[0][b_off + 8192]);
    if (grp == 1) __syncthreads();                    // group 1 runs half a step behind group 0

    for (int t = 0; t < ntiles; ++t) {
      // ---- MFMA half: step t's key tile from stage t % PF2_NSTAGE
      const char* kb = &ktile[t & (PF2_NSTAGE - 1)][b_off];
      f32x16 acc[2][2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) acc[c][rt] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bf16x8 n0 = b0, n1 = b1;
        if (kk + 1 < 8) {
          n0 = *(const bf16x8*)(kb + (kk + 1) * 512);
          n1 = *(const bf16x8*)(kb + 8192 + (kk + 1) * 512);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          acc[0][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][kk], b0, acc[0][rt], 0, 0, 0);
          acc[1][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][kk], b1, acc[1][rt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        b0 = n0;
        b1 = n1;
      }
      // Group 0: this wave's share of tile t + 1 landed (its requests for
      // t + 2, the last vector-memory instructions it issued, may still fly).
      // Group 1: its share of tile t + 2 landed as well, before the barrier
      // that ends group 0's MFMA half t + 1: group 0 reads tile t + 2's first
      // B operands at the end of its VALU half t + 1.
      if (t < t_part) wait_vmcnt<NB>(); else wait_vmcnt<0>();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);               // the VALU half stays after the barrier
      // ---- VALU half: reduce step t, offer it, request the tile three steps ahead
      float part2[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float ps = 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int i = 0; i < 16; ++i) ps = __builtin_fmaf(wl[rt][i], relu(acc[c][rt][i]), ps);
        part2[c] = ps;
      }
      // The score is never -0.0: each partial sum starts as fma(w, r, +0) with
      // r >= +0, so it is +0 or non-zero, and later fmas and the final add
      // return -0.0 only from two -0.0 operands.
      // The next MFMA half's first B operands, read here so that the offer
      // hides their latency: tile t + 1 is whole in LDS (both groups' shares
      // landed before the barrier that began this half).
      if (t + 1 < ntiles) {
        const char* kn = &ktile[(t + 1) & (PF2_NSTAGE - 1)][b_off];
        b0 = *(const bf16x8*)(kn);
        b1 = *(const bf16x8*)(kn + 8192);
      }
      const float score = half_swap_sum(part2[0], part2[1]);
      const u64 key = ((u64)order_bits_nz(score) << 32) | (u64)(nidx0 - (uint32_t)t * tile_step);
      key_offer<MODE>(st, key, l < vis - t * PF_KTILE, a, hist, list);
      // stage (t + 3) % 4 last held step t - 1, whose readers passed a barrier before this half began
      if (t + PF2_NSTAGE - 1 < ntiles) load_tile(t + PF2_NSTAGE - 1, (t + PF2_NSTAGE - 1) & (PF2_NSTAGE - 1), knext);
      knext += tile_bytes;
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);               // the next MFMA half stays after the barrier
    }
    if (grp == 0) __syncthreads();                    // both groups pass the same number of barriers
    Slot fs;
    fs.cand = st.cand;
    fs.cnt = st.cnt;
    fs.surv = st.surv;
    fs.lo = order_bits_score(st.lo_o);
    fs.hi = order_bits_score(st.hi_o);
    finish_row<MODE>(a, fs, b, row, part, hist, list);
  }
}

// ============================================================ generic prefill
//
// Any H, D and dtype (fp32 or bf16): each lane computes one (query, key)
// score with fp32 FMAs in index order (exact for small-integer inputs).  No
// workgroup barriers: waves are independent.

template <typename Tin>
__device__ __forceinline__ float ld_f32(const Tin* p, size_t i);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_f32<__bf16>(const __bf16* p, size_t i) { return (float)p[i]; }

template <int MODE, typename Tin>
__global__ __launch_bounds__(PF_THREADS) void prefill_generic_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t hist_all[PF_THREADS / WAVE][SEL_BINS];
  __shared__ u64 list_all[PF_THREADS / WAVE][WAVE_LIST];
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  uint32_t* hist = hist_all[wv];
  u64* list = list_all[wv];
  const Tin* Q = (const Tin*)a.q;
  const Tin* K = (const Tin*)a.k;

  for (int r = 0;; ++r) {
    const int it = round_item(r);
    if (r * (int)gridDim.x >= a.n_items) break;
    if (it >= a.n_items) continue;
    int b, qb, part;
    decode_item(a, it, b, qb, part);
    int vis_max;
    const bool need = block_needs_scores<MODE>(a, b, qb, part, vis_max);
    const int row = qb * PF_ROWS + wv;
    const int vis = row_visible(a, b, row, part);
    if (row >= a.S_q) continue;
    if (!need) {
      wave_emit_all_visible(a, b, row, part, vis);
      continue;
    }
    Slot st;
    slot_init(st, a.cand + ((size_t)blockIdx.x * PF_ROWS + wv) * a.C, a, MODE);
    const size_t qoff = ((size_t)b * a.S_q + row) * a.H;
    for (int j0 = 0; j0 < vis; j0 += WAVE) {
      const int j = j0 + l;
      const bool valid = j < vis;
      float score = 0.f;
      uint32_t s_idx = 0;
      if (valid) {
        s_idx = (uint32_t)(part + a.P * j);
        const size_t koff = ((size_t)b * a.T + s_idx) * a.D;
        for (int h = 0; h < a.H; ++h) {
          float dot = 0.f;
          const size_t qh = (qoff + h) * a.D;
          for (int d = 0; d < a.D; ++d) dot = __builtin_fmaf(ld_f32(Q, qh + d), ld_f32(K, koff + d), dot);
          score = __builtin_fmaf(a.w[qoff + h], relu(dot), score);
        }
      }
      wave_offer<MODE>(st, score, s_idx, valid, a, hist, list);
    }
    finish_row<MODE>(a, st, b, row, part, hist, list);
  }
}

// ============================================================ decode
//
// decode_score: grid (nsplit, B*S_q).  Workgroup x scans keys
// [x*chunk, (x+1)*chunk) of one query row; each wave takes 32-key steps.  The
// key rows are read whole from HBM and reach the MFMA B operands through a
// per-wave LDS tile; the query's 64x128 A operand sits in LDS and the lane's
// head weights in registers.

// Slot of 16-byte piece p (0..15) of key c (0..31) in a per-wave 8 KB tile
// of 32 key rows: the row-wise writes and the column-wise MFMA B-operand reads
// of 16 lanes both cover all banks.
__device__ __forceinline__ int key_tile_slot(int c, int p) { return 16 * c + (p ^ (c & 15)); }

__device__ __forceinline__ int decode_visible(const DecodeArgs& a, int b, int i) {
  long long v = a.causal ? (a.q_pos0 + i) / a.m + 1 : (long long)a.T;
  if (v > a.T) v = a.T;
  if (a.kv_len) {
    long long kv = a.kv_len[b];
    if (kv < 0) kv = 0;
    if (v > kv) v = kv;
  }
  return (int)v;
}

template <int CH>
__device__ __forceinline__ void decode_score_body(const DecodeArgs& a) {
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int row = blockIdx.y, b = row / a.S_q, i = row % a.S_q;
  const int vis = decode_visible(a, b, i);
  const int start = blockIdx.x * CH;
  const int end = start + CH < vis ? start + CH : vis;
  if (start >= end) return;
  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  // The query's 64x128 A operand lives in LDS in MFMA lane order (each wave
  // copies two of the eight 16-deep slices; 16-byte reads without bank
  // conflicts), which leaves the registers for a ring of DEC_RING key-row
  // buffers: DEC_RING - 1 steps (8 KB each per wave) stay in flight.
  // Key rows are read whole (1 KB of consecutive bytes per load instruction,
  // with the non-temporal hint: each byte is used once) and pass through a
  // per-wave LDS tile into the MFMA B layout.  In the tile, 16-byte piece p
  // of step key c sits at slot 16c + (p ^ (c % 16)), so both the row-wise
  // writes and the column-wise operand reads of 16 lanes spread over all
  // banks.
  __shared__ bf16x8 Als[2][8][WAVE];
  __shared__ u32x4 Kls[DEC_THREADS / WAVE][32 * 16];
  float* out = a.scores + (size_t)row * dec_row_floats(a.T);
  const size_t kseq = (size_t)b * a.T;
  constexpr int STEP = 32, STRIDE = STEP * (DEC_THREADS / WAVE);
  // Instruction i of a step reads keys base + 4i .. +3: lane l takes piece
  // l % 16 of key base + 4i + l / 16.
  auto load = [&](int base, u32x4 (&bf)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int s = base + 4 * i + (l >> 4);
      s = s < end ? s : end - 1;
      bf[i] = __builtin_nontemporal_load((const u32x4*)(K + (kseq + s) * MD) + (l & 15));
    }
  };
  u32x4* kt = Kls[wv];
  static_assert(CH % STRIDE == 0, "decode chunk must be whole steps");
  static_assert(DEC_THREADS / WAVE * 2 == 8, "each wave copies two query slices");
  constexpr int NSTEP = CH / STRIDE;
  const int base0 = start + STEP * wv;
  bf16x8 qa[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const bf16x8* src = (const bf16x8*)(Q + ((size_t)row * MH + rt * 32 + (l & 31)) * MD);
#pragma unroll
    for (int h = 0; h < 2; ++h) qa[rt][h] = src[2 * (2 * wv + h) + (l >> 5)];
  }
  u32x4 bb[DEC_RING][8];
#pragma unroll
  for (int st = 0; st < DEC_RING - 1; ++st) load(base0 + st * STRIDE, bb[st]);
  float wl[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e) wl[rt][e] = a.w[(size_t)row * MH + rt * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3)];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int h = 0; h < 2; ++h) Als[rt][2 * wv + h][l] = qa[rt][h];
  __syncthreads();
  // Steps are a compile-time count, so the loop unrolls completely: a ring of
  // DEC_RING buffers without register copies, and exact wait counts for the
  // prefetched rows because scores stay in registers until the loop ends.
  float sc[NSTEP];
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {
    if (st + DEC_RING - 1 < NSTEP) load(base0 + (st + DEC_RING - 1) * STRIDE, bb[(st + DEC_RING - 1) % DEC_RING]);
    asm volatile("" ::: "memory");                    // re-read the A slices from LDS every step
    __builtin_amdgcn_sched_barrier(0);
    // the step's rows into the tile, then B operands: lane l holds 16 bytes
    // (d = 8 * (2 * kk + l / 32) .. + 7) of key l % 32; a wave's LDS accesses
    // complete in order, so the tile is reused without a barrier
#pragma unroll
    for (int i = 0; i < 8; ++i) kt[key_tile_slot(4 * i + (l >> 4), l & 15)] = bb[st % DEC_RING][i];
    bf16x8 bk[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) bk[kk] = __builtin_bit_cast(bf16x8, kt[key_tile_slot(l & 31, 2 * kk + (l >> 5))]);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Als[rt][kk][l], bk[kk], acc[rt], 0, 0, 0);
    float ps = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int e = 0; e < 16; ++e) ps = __builtin_fmaf(wl[rt][e], relu(acc[rt][e]), ps);
    sc[st] = half_swap_sum(ps, ps);                   // both halves: the full score of key (l & 31)
  }
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {               // no branch: keys past the end go to the row's pad
    const int s = base0 + st * STRIDE + (l & 31);
    out[s < end ? s : a.T + (l & 31)] = sc[st];       // lanes l and l^32 store the same value
  }
  // Selection bound of this wave for decode_select_kernel: order bits P and a
  // count c such that at least c of the wave's keys have order bits >= P.  The
  // row's k is spread over the waves of its whole chunks as a target g per
  // wave (so the counts of those waves alone reach k); P is the largest value
  // with g of the lanes' two best scores at or above it, settled one bit at a
  // time from ballot counts.  A wave that cannot vouch for g keys that way
  // (a partial chunk, or g above two keys per lane) reports its smallest
  // score and all of its keys.
  {
    constexpr u64 LO = 0xFFFFFFFFull;                  // lanes 32-63 repeat lanes 0-31
    constexpr int WPC = DEC_THREADS / WAVE;            // waves per chunk
    const int nfull = vis / CH * WPC;                  // waves with all CH / WPC keys
    const int g = nfull > 0 ? (a.kk + nfull - 1) / nfull : 0x7FFFFFFF;
    uint32_t t1 = 0u, t2 = 0u, mn = ~0u;               // 0 is below every score's order bits
    int nv = 0;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const bool ok = base0 + st * STRIDE + (l & 31) < end;
      const uint32_t o = ok ? score_order_bits(sc[st]) : 0u;
      t2 = max(t2, min(t1, o));
      t1 = max(t1, o);
      mn = ok ? min(mn, o) : mn;
      nv += __popcll(ballot(ok) & LO);
    }
    auto count_ge = [&](uint32_t c) { return __popcll(ballot(t1 >= c) & LO) + __popcll(ballot(t2 >= c) & LO); };
    uint32_t P = ~0u;
    int c = 0;
    if (g <= 64 && count_ge(1u) >= g) {
      P = 0u;
      for (int bit = 31; bit >= 16; --bit)            // 16 bits: within 1/128 of the exact value
        if (count_ge(P | (1u << bit)) >= g) P |= 1u << bit;
      c = count_ge(P);
    } else if (nv > 0) {
      P = wave_min_u32(mn);
      c = nv;
    }
    const uint32_t mx = wave_max_u32(t1);
    if (l == 0) a.bounds[(size_t)row * a.nbw + blockIdx.x * WPC + wv] = make_uint4(P, (uint32_t)c, mx, 0u);
  }
}

template <int CH>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode_score_kernel(DecodeArgs a) { decode_score_body<CH>(a); }

// Several problems of one shape in one launch (grid z = problem).
template <int CH>
__global__ __launch_bounds__(DEC_THREADS, 2) void decode_score_batch_kernel(DecodeBatch bt) {
  decode_score_body<CH>(bt.a[blockIdx.z]);
}

// decode_select: one workgroup per query row; exact top-kk of the row's
// dense scores.  Wave w holds the contiguous element range [w*2048, w*2048+2048)
// in registers (lane l's v[4i .. 4i+3] are elements w*2048 + 256*i + 4*l .. +3,
// read with one 16-byte load).
//
// The scan's per-wave bounds give L = min_w P_w with at least sum_w c_w >= kk
// keys at or above it, so the kk-th largest key scores >= L and only keys
// scoring >= L (about a tenth of a row of i.i.d. scores) are candidates.  One
// pass over the registers packs each wave's candidates, in element order, into
// the wave's LDS segment (the register passes cost VALU time on one CU for
// every element, so there is only one).  The candidates are histogrammed; keys
// in bins above the one holding rank kk are emitted in segment order, and the
// keys of that bin, gathered into an LDS list, are ranked against each other
// (one thread per key) and the best r emitted in rank order: deterministic
// output with four block barriers.  Rows the bounds cannot narrow (no bound,
// equal scores, a full segment, a crowded bin) and rows longer than the
// registers hold take the select over the dense scores in memory.
constexpr int DEC_REG = 32;                              // keys per lane: rows up to 32768 in registers
constexpr int DEC_LIST = 256;                            // boundary-bin keys ranked directly
constexpr int DEC_SEG = 512;                             // candidate slots per wave (of its 2048 elements)

// Bins for candidate keys whose scores lie in [lo, hi]: on the score's order
// bits (a fixed number of bins per binade, so a few far outliers at the top do
// not crowd the bulk near lo into one bin) when the candidates are positive
// and span at most 20 binades, else linear in the score (finer near lo once
// the order-bit bins would each cover a large part of a binade).  Both are
// monotone in the key.
struct RowBins {
  bool ord;
  uint32_t base;
  int shift;
  LinBins lin;
  __device__ __forceinline__ int operator()(u64 key) const {
    if (ord) {
      const uint32_t b = ((uint32_t)(key >> 32) - base) >> shift;
      return (int)(b < (uint32_t)(SEL_BINS - 1) ? b : (uint32_t)(SEL_BINS - 1));
    }
    return lin(key);
  }
};

__device__ __forceinline__ bool row_bins_ok(uint32_t lo_bits, uint32_t hi_bits, RowBins& rb) {
  const float lo = order_bits_score(lo_bits), hi = order_bits_score(hi_bits);
  rb.ord = lo > 0.f && hi < 1048576.f * lo;
  rb.base = lo_bits;
  const uint32_t span = hi_bits - lo_bits;
  const int bits = span ? 32 - __clz((int)span) : 0;
  rb.shift = bits > SEL_RB ? bits - SEL_RB : 0;
  if (rb.ord) return span != 0u;
  return lin_bins_ok(lo, hi, rb.lin);
}

__device__ __forceinline__ void decode_select_body(const DecodeArgs& a) {
  constexpr int NW = DEC_SEL_THREADS / WAVE;
  __shared__ __attribute__((aligned(16))) uint32_t hist[SEL_BINS];
  __shared__ u64 red[2 * NW];
  __shared__ u64 list[DEC_LIST];
  __shared__ float segv_all[NW * DEC_SEG];            // candidate scores and indices, per wave
  __shared__ uint32_t segi_all[NW * DEC_SEG];
  __shared__ uint32_t part[3 * NW];
  __shared__ int wcnt[NW];
  __shared__ int lcnt;
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int row = blockIdx.x, b = row / a.S_q, i = row % a.S_q;
  const int vis = decode_visible(a, b, i);
  const float* sc = a.scores + (size_t)row * dec_row_floats(a.T);
  int32_t* oi = a.out_idx + (size_t)row * a.kk;
  float* os = a.out_score ? a.out_score + (size_t)row * a.kk : nullptr;
  float* segv = segv_all + wv * DEC_SEG;
  uint32_t* segi = segi_all + wv * DEC_SEG;
  auto seg = [&](int e) { return make_key(segv[e], segi[e]); };
  int w = 0;
  bool dense = vis > DEC_REG * DEC_SEL_THREADS;
  if (!dense) {
    // v[j] holds element el(j): lane l loads the 4 consecutive elements
    // wv * 2048 + 256 * (j / 4) + 4 * l .. + 3 with one 16-byte load (a load
    // instruction brings 1 KB of the row).
    const int e0 = wv * (DEC_REG * WAVE) + 4 * l;
    auto el = [&](int j) { return e0 + (j >> 2) * (4 * WAVE) + (j & 3); };
    // the row's bounds first: loads complete in order, so reducing them does
    // not wait for the score loads behind them
    const int nwr = (vis + a.chunk - 1) / a.chunk * (DEC_THREADS / WAVE);   // <= 128 here
    const uint4 bd = tid < nwr && vis > a.kk ? a.bounds[(size_t)row * a.nbw + tid] : make_uint4(~0u, 0u, 0u, 0u);
    float v[DEC_REG];
    const int glast = vis > 0 ? (vis - 1) & ~3 : 0;   // last group holding a visible element
#pragma unroll
    for (int j = 0; j < DEC_REG; j += 4) {            // every load in flight at once; a group
      const int g = el(j);                            // past the row's end re-reads the last one
      const float4 t = *(const float4*)(sc + (g < glast ? g : glast));   // (its elements are masked)
      v[j] = t.x; v[j + 1] = t.y; v[j + 2] = t.z; v[j + 3] = t.w;
    }
    // Threshold mode: the survivors are the keys >= thr_fixed, i.e. scoring
    // >= sf (the smallest fp32 score above the threshold; the float compare
    // agrees with the order bits, -0 included).  Their count is written out;
    // when it exceeds kk (the cap) the survivors' best kk are the row's top kk
    // and the top-k select below runs unchanged.
    const bool thr = a.thr_fixed != 0ull;
    const float sf = thr ? key_score(a.thr_fixed) : -__builtin_inff();
    bool all = vis <= a.kk;
    if (thr) {
      int mine = 0;
#pragma unroll
      for (int j = 0; j < DEC_REG; ++j) mine += __popcll(ballot(el(j) < vis && v[j] >= sf));
      if (l == 0) wcnt[wv] = mine;
      __syncthreads();
      int tot = 0;
      for (int j = 0; j < NW; ++j) tot += wcnt[j];
      if (tid == 0) a.out_count[row] = tot;
      all = tot <= a.kk;
      __syncthreads();                                // wcnt is reused below
    }
    if (all) {                                        // every visible key (survivor), in element order
      int mine = 0;
#pragma unroll
      for (int j = 0; j < DEC_REG; ++j) mine += __popcll(ballot(el(j) < vis && v[j] >= sf));
      if (l == 0) wcnt[wv] = mine;
      __syncthreads();
      int off = 0, tot = 0;
      for (int j = 0; j < NW; ++j) {
        off += j < wv ? wcnt[j] : 0;
        tot += wcnt[j];
      }
#pragma unroll
      for (int j = 0; j < DEC_REG; ++j) {
        const int s = el(j);
        const bool keep = s < vis && v[j] >= sf;
        const u64 m = ballot(keep);
        if (keep) emit_key(make_key(v[j], (uint32_t)s), off + lanes_below(m), a.kk, oi, os);
        off += __popcll(m);
      }
      w = tot;
    } else {
      // [1] bounds -> L (order bits), their count, row max; clear the histogram meanwhile
      const uint32_t P0 = wave_min_u32(bd.y ? bd.x : ~0u);
      const int c0 = wave_sum_i32((int)bd.y);
      const uint32_t M0 = wave_max_u32(bd.z);
      if (l == 0) { part[wv] = P0; part[NW + wv] = (uint32_t)c0; part[2 * NW + wv] = M0; }
      for (int e = 4 * tid; e < SEL_BINS; e += 4 * DEC_SEL_THREADS) *(uint4*)&hist[e] = make_uint4(0u, 0u, 0u, 0u);
      if (tid == 0) lcnt = 0;
      __syncthreads();
      uint32_t P = ~0u, M = 0u;
      long long cs = 0;
      for (int j = 0; j < NW; ++j) {
        P = min(P, part[j]);
        cs += part[NW + j];
        M = max(M, part[2 * NW + j]);
      }
      RowBins rb;
      const float lf = order_bits_score(P);
      bool fast = cs >= a.kk && row_bins_ok(P, M, rb);
      int cw = 0, bin = 0, r = 0;
      if (fast) {
        // [2] the one register pass: pack candidates (score >= L; the float
        // compare agrees with the order bits, -0 included) into this wave's
        // segment, then histogram the segment
        // (score and index as two 32-bit words: no key is formed per element,
        // and a wave whose whole range is visible skips the range test)
        auto pack = [&](auto in_range) {
#pragma unroll
          for (int j = 0; j < DEC_REG; ++j) {
            const int s = el(j);
            const bool c = in_range(s) && v[j] >= lf;
            const u64 m = ballot(c);
            const int pos = cw + lanes_below(m);
            if (c && pos < DEC_SEG) { segv[pos] = v[j]; segi[pos] = (uint32_t)s; }
            cw += __popcll(m);
          }
        };
        if ((wv + 1) * DEC_REG * WAVE <= vis) pack([](int) { return true; });
        else pack([&](int s) { return s < vis; });
        wave_lds_sync();
        const int cn = cw < DEC_SEG ? cw : DEC_SEG;
        for (int e = l; e < cn; e += WAVE) atomicAdd(&hist[rb(seg(e))], 1u);
        if (l == 0) wcnt[wv] = cw;
        __syncthreads();
        int mx = 0;
        for (int j = 0; j < NW; ++j) mx = max(mx, wcnt[j]);
        fast = mx <= DEC_SEG;
      }
      if (fast) {
        // [3] the bin holding rank kk
        if (wv == 0) {
          const BinPick pk = wave_pick_bin(hist, SEL_BINS, a.kk);
          if (l == 0) { red[0] = (u64)pk.bin; red[1] = (u64)pk.above; red[2] = (u64)pk.count; }
        }
        __syncthreads();
        bin = (int)red[0];
        r = a.kk - (int)red[1];
        const int bcnt = (int)red[2];
        fast = bcnt > 0 && bcnt <= DEC_LIST;
      }
      if (fast) {
        // [4] gather the boundary bin; count this wave's keys above it
        int up = 0;
        for (int e00 = 0; e00 < cw; e00 += WAVE) {
          const int e = e00 + l;
          const u64 x = e < cw ? seg(e) : 0ull;
          const int bx = e < cw ? rb(x) : -1;
          up += __popcll(ballot(bx > bin));
          if (bx == bin) list[atomicAdd(&lcnt, 1)] = x;
        }
        if (l == 0) red[4 + wv] = (u64)up;
        __syncthreads();
        // [5] keys above the bin, in segment order ...
        int off = 0;
        for (int j = 0; j < wv; ++j) off += (int)red[4 + j];
        for (int e00 = 0; e00 < cw; e00 += WAVE) {
          const int e = e00 + l;
          const u64 x = e < cw ? seg(e) : 0ull;
          const bool keep = e < cw && rb(x) > bin;
          const u64 m = ballot(keep);
          if (keep) emit_key(x, off + lanes_below(m), a.kk, oi, os);
          off += __popcll(m);
        }
        // ... and the bin's best r, each placed by its rank within the bin
        const int bc = lcnt, above = a.kk - r;
        if (tid < bc) {
          const u64 x = list[tid];
          int g = 0;
#pragma unroll 8
          for (int q = 0; q < bc; ++q) g += list[q] > x ? 1 : 0;
          if (g < r) emit_key(x, above + g, a.kk, oi, os);
        }
        w = a.kk;
      } else {
        dense = true;
      }
    }
  }
  if (dense) {                                        // uniform: every decision above came from LDS
    __syncthreads();
    u64 T = 0ull;
    if (a.thr_fixed != 0ull && vis > DEC_REG * DEC_SEL_THREADS) {   // threshold mode, long row: count first
      int mine = 0;
      for (int s = tid; s < vis; s += DEC_SEL_THREADS) mine += make_key(sc[s], (uint32_t)s) >= a.thr_fixed;
      mine = wave_sum_i32(mine);
      if (l == 0) wcnt[wv] = mine;
      __syncthreads();
      int tot = 0;
      for (int j = 0; j < NW; ++j) tot += wcnt[j];
      if (tid == 0) a.out_count[row] = tot;
      __syncthreads();
      if (tot <= a.kk) T = a.thr_fixed;
    }
    if (T == 0ull) T = block_select_kth_dense<DEC_SEL_THREADS>(sc, vis, a.kk, hist, red);
    for (int base = 0; base < vis; base += DEC_SEL_THREADS) {
      const int s = base + tid;
      const u64 x = s < vis ? make_key(sc[s], (uint32_t)s) : 0ull;
      const bool keep = s < vis && x >= T;
      const u64 m = ballot(keep);
      if (l == 0) wcnt[wv] = __popcll(m);
      __syncthreads();
      int off = 0, tot = 0;
      for (int j = 0; j < NW; ++j) {
        off += j < wv ? wcnt[j] : 0;
        tot += wcnt[j];
      }
      if (keep) emit_key(x, w + off + lanes_below(m), a.kk, oi, os);
      w += tot;
      __syncthreads();
    }
  }
  w = w < a.kk ? w : a.kk;
  for (int e = w + tid; e < a.kk; e += DEC_SEL_THREADS) {
    oi[e] = -1;
    if (os) os[e] = -__builtin_inff();
  }
}

__global__ __launch_bounds__(DEC_SEL_THREADS) void decode_select_kernel(DecodeArgs a) { decode_select_body(a); }

__global__ __launch_bounds__(DEC_SEL_THREADS) void decode_select_batch_kernel(DecodeBatch bt) {
  decode_select_body(bt.a[blockIdx.z]);
}

// ============================================================ sparse attention
//
// CSA stage 4: every query head attends, with scaled softmax, to the key and
// value rows its row of indices selects (the indexer's output); entries
// outside [0, T) are skipped.  H = 64 heads, Dk = Dv = 128, bf16 inputs,
// fp32 accumulation and output.
//
// attn_chunk_kernel: grid (nsplit, rows), 8 waves.  A workgroup takes the
// row's AT_CHUNK-entry (256) chunks split, split + nsplit, ... with an online
// softmax.  Per chunk: wave w gathers the key rows of entries 32w..32w+31
// straight into MFMA B operands (16 B per lane), while every thread gathers
// its share of the chunk's value rows, all in flight together; wave w forms
// the 64 x 32 logits of its entries with the query slices (LDS, A operand);
// the chunk's per-head max and the running max come through LDS; p =
// exp(z - m) goes to LDS as bf16 in the MFMA A layout, the value rows go to
// LDS transposed (dv-major), and wave w then accumulates head tile w % 2 for
// output columns 32 * (w / 2) .. + 31 with P.V MFMAs after rescaling them by
// exp(m_old - m_new).  Both LDS tiles are XOR-swizzled in 16-byte pieces
// (piece ^ row % 16) so that the 16-byte operand reads of 32 rows at the same
// piece spread over the banks.
// attn_combine_kernel merges the nsplit partial results of a row.

// Lane exchanges inside 16-lane rows through DPP (no LDS round trip):
// quad_perm [1,0,3,2] and [2,3,0,1], then the mirrored half row and row, pair
// every lane with one whose partial covers the other lanes of its 2, 4, 8 and
// 16 group; the last step (lane ^ 16) crosses rows with v_permlane16_swap.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

// The step between 16-lane rows (lane ^ 16): v_permlane16_swap with x in both
// operands exchanges rows 1 and 3 of the first with rows 0 and 2 of the
// second, so every lane ends with its own row's value in one result and the
// neighbouring row's in the other; their max or sum is the butterfly step,
// without an LDS round trip.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t at_swz(int r, int col) {   // bf16 element (r, col) of a 128-wide tile
  return (uint32_t)(r * AT_CHUNK * 2 + ((((col >> 3) ^ (r & 15)) << 4) | ((col & 7) << 1)));
}

__global__ __launch_bounds__(AT_THREADS, 1) void attn_chunk_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char ps[AT_H * AT_CHUNK * 2];      // P (bf16), head-major
  __shared__ __attribute__((aligned(16))) char vt[AT_D * AT_CHUNK * 2];      // V^T (bf16), dv-major
  __shared__ bf16x8 qs[2][8][WAVE];                                          // Q in MFMA A-operand order
  constexpr int NWV = AT_THREADS / WAVE;
  __shared__ float red[NWV][AT_H];
  __shared__ float mrun[AT_H], lrun[AT_H], mnew_s[AT_H], alpha_s[AT_H];
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int row = blockIdx.y, split = blockIdx.x, b = row / a.S_q;
  const int nchunk = (a.n_sel + AT_CHUNK - 1) / AT_CHUNK;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;
  const int32_t* irow = a.idx + (size_t)row * a.n_sel;
  const size_t kseq = (size_t)b * a.T;

  // index entries of this lane's key column and of this thread's two value
  // rows (2p, 2p+1 with p = tid / 4; columns 32 * (tid % 4) .. + 31), for the
  // first chunk here and for the next one at the end of each step
  auto entry = [&](int j) { return j < a.n_sel ? irow[j] : -1; };
  int ik = entry(split * AT_CHUNK + 32 * wv + (l & 31));
  int iv0 = entry(split * AT_CHUNK + 2 * (tid >> 2)), iv1 = entry(split * AT_CHUNK + 2 * (tid >> 2) + 1);
  // the query operand goes to LDS (wave w copies slice w of both head
  // halves), which leaves registers for the key and value rows of a chunk in
  // flight together; it is stored there once the first chunk's rows have been
  // requested
  static_assert(AT_THREADS / WAVE == 8, "one query slice per wave");
  bf16x8 qv[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const bf16x8* src = (const bf16x8*)((const __bf16*)a.q + ((size_t)row * AT_H + rt * 32 + (l & 31)) * AT_D);
    qv[rt] = src[2 * wv + (l >> 5)];
  }
  if (tid < AT_H) {
    mrun[tid] = -__builtin_inff();
    lrun[tid] = 0.f;
  }
  // P.V roles: wave w accumulates head tile rt = w % 2 for output columns
  // 32 * (w / 2) .. + 31
  const int prt = wv & 1, pdc = 32 * (wv >> 1);
  f32x16 o = f32x16{};
  // head row of accumulator element e (rows of tile rt are rt*32 + this)
  auto hrow = [&](int e) { return 8 * (e >> 2) + 4 * (l >> 5) + (e & 3); };

  for (int c = split; c < nchunk; c += a.nsplit) {
    const bool vk = ik >= 0 && ik < a.T;
    const bool vv0 = iv0 >= 0 && iv0 < a.T, vv1 = iv1 >= 0 && iv1 < a.T;
    bf16x8 bk[8], vr[2][4];
    {                                                   // the chunk's key and value rows, all in flight
      const bf16x8* src = (const bf16x8*)(K + (kseq + (vk ? ik : 0)) * AT_D);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) bk[kk] = src[2 * kk + (l >> 5)];
      const bf16x8* v0 = (const bf16x8*)(V + (kseq + (vv0 ? iv0 : 0)) * AT_D + (tid & 3) * 32);
      const bf16x8* v1 = (const bf16x8*)(V + (kseq + (vv1 ? iv1 : 0)) * AT_D + (tid & 3) * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vr[0][i] = v0[i];
        vr[1][i] = v1[i];
      }
    }
    if (c == split) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) qs[rt][wv][l] = qv[rt];
    }
    __syncthreads();                                    // the query slices are in LDS (first chunk)
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qs[rt][kk][l], bk[kk], acc[rt], 0, 0, 0);
    // scaled logits; skipped entries at -inf; per-head max over the wave's 32
    // entries (the 32 butterflies run side by side, one exchange step at a
    // time, so that their lane exchanges overlap instead of waiting in turn)
    float red_v[16];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[rt][e] = vk ? a.scale * acc[rt][e] : -__builtin_inff();   // the logit, in place
        red_v[e] = acc[rt][e];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = fmaxf(red_v[e], dpp_f32<DPP_XOR1>(red_v[e]));
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = fmaxf(red_v[e], dpp_f32<DPP_XOR2>(red_v[e]));
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = fmaxf(red_v[e], dpp_f32<DPP_HALF_MIRROR>(red_v[e]));
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = fmaxf(red_v[e], dpp_f32<DPP_MIRROR>(red_v[e]));
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = max_xor16(red_v[e]);
      if ((l & 31) == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wv][rt * 32 + hrow(e)] = red_v[e];
      }
    }
    __syncthreads();
    if (tid < AT_H) {
      float cm = red[0][tid];
#pragma unroll
      for (int j = 1; j < NWV; ++j) cm = fmaxf(cm, red[j][tid]);
      const float mo = mrun[tid], mn = fmaxf(mo, cm);
      mnew_s[tid] = mn;
      alpha_s[tid] = mn == -__builtin_inff() ? 1.f : __expf(mo - mn);
    }
    __syncthreads();
    // p = exp(z - m_new) to LDS (bf16, A layout); per-head sums of the wave's p
    // (of the rounded values the P.V product uses), butterflies side by side
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int h = rt * 32 + hrow(e);
        const float mn = mnew_s[h];
        const float pv = mn == -__builtin_inff() ? 0.f : __expf(acc[rt][e] - mn);
        const __bf16 pb = (__bf16)pv;
        *(__bf16*)(ps + at_swz(h, 32 * wv + (l & 31))) = pb;
        red_v[e] = (float)pb;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] += dpp_f32<DPP_XOR1>(red_v[e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] += dpp_f32<DPP_XOR2>(red_v[e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] += dpp_f32<DPP_HALF_MIRROR>(red_v[e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] += dpp_f32<DPP_MIRROR>(red_v[e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) red_v[e] = add_xor16(red_v[e]);
      if ((l & 31) == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wv][rt * 32 + hrow(e)] = red_v[e];
      }
    }
    // value rows 2p, 2p+1 (columns 32 * (tid % 4) .. + 31), transposed: one
    // 4-byte store per column holds both rows.  The pairs are formed on the
    // 32-bit words (column 2u in the low half of word u, 2u+1 in the high half).
    {
      const int kcol = 2 * (tid >> 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w0 = __builtin_bit_cast(u32x4, vr[0][i]), w1 = __builtin_bit_cast(u32x4, vr[1][i]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int col = (tid & 3) * 32 + 8 * i + 2 * u;
          *(uint32_t*)(vt + at_swz(col, kcol)) = (w0[u] & 0xFFFFu) | (w1[u] << 16);
          *(uint32_t*)(vt + at_swz(col + 1, kcol)) = (w0[u] >> 16) | (w1[u] & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();
    if (tid < AT_H) {
      float cs = 0.f;
#pragma unroll
      for (int j = 0; j < NWV; ++j) cs += red[j][tid];
      lrun[tid] = alpha_s[tid] * lrun[tid] + cs;
      mrun[tid] = mnew_s[tid];
    }
    // rescale this wave's output columns, then O += P . V over the chunk
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] *= alpha_s[prt * 32 + hrow(e)];
#pragma unroll
    for (int ks = 0; ks < AT_CHUNK / 16; ++ks) {
      const int kc = 16 * ks + 8 * (l >> 5);
      const bf16x8 bv = *(const bf16x8*)(vt + at_swz(pdc + (l & 31), kc));
      const bf16x8 ap = *(const bf16x8*)(ps + at_swz(prt * 32 + (l & 31), kc));
      o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap, bv, o, 0, 0, 0);
    }
    const int cn = c + a.nsplit;                        // the next chunk's entries
    ik = entry(cn * AT_CHUNK + 32 * wv + (l & 31));
    iv0 = entry(cn * AT_CHUNK + 2 * (tid >> 2));
    iv1 = entry(cn * AT_CHUNK + 2 * (tid >> 2) + 1);
    __syncthreads();                                    // P, V^T and the stats are reused by the next chunk
  }
  const size_t pr = (size_t)row * a.nsplit + split;
  float* op = a.opart + pr * AT_H * AT_D;
#pragma unroll
  for (int e = 0; e < 16; ++e) op[(size_t)(prt * 32 + hrow(e)) * AT_D + pdc + (l & 31)] = o[e];
  if (tid < AT_H) {
    a.mpart[pr * AT_H + tid] = mrun[tid];
    a.lpart[pr * AT_H + tid] = lrun[tid];
  }
}

// One workgroup per (head, query row), one thread per output column:
// o = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s over the row's partial
// results (0 where no entry was valid).
__global__ __launch_bounds__(AT_D) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, row = blockIdx.y, x = threadIdx.x;
  const size_t pr0 = (size_t)row * a.nsplit;
  float M = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.mpart[(pr0 + s) * AT_H + h]);
  float num = 0.f, den = 0.f;
  if (M != -__builtin_inff()) {
#pragma unroll 8
    for (int s = 0; s < a.nsplit; ++s) {
      const float ms = a.mpart[(pr0 + s) * AT_H + h];
      const float f = ms == -__builtin_inff() ? 0.f : __expf(ms - M);
      num += f * a.opart[((pr0 + s) * AT_H + h) * AT_D + x];
      den += f * a.lpart[(pr0 + s) * AT_H + h];
    }
  }
  a.out[((size_t)row * AT_H + h) * AT_D + x] = den > 0.f ? num / den : 0.f;
}

// ============================================================ union of selections
//
// Multi-layer selection (FlashMemory's Memory Indexer on three layers whose
// decisions are OR-ed while decoding): per row, the union of L index lists.
// One workgroup per row marks every valid entry (0 <= v < T) in an LDS bitmap
// of T bits, then thread t takes a contiguous run of bitmap words, counts its
// bits, and after a block-wide prefix sum writes its indices in ascending
// order: the union sorted by index, deterministic.

__global__ __launch_bounds__(UN_THREADS) void union_rows_kernel(UnionArgs a) {
  __shared__ uint32_t words[UN_MAX_T / 32];
  __shared__ int wsum[UN_THREADS / WAVE];
  constexpr int NW = UN_THREADS / WAVE;
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const long long row = blockIdx.x;
  const int nwords = (a.T + 31) / 32;
  for (int i = tid; i < nwords; i += UN_THREADS) words[i] = 0u;
  __syncthreads();
  for (int li = 0; li < a.L; ++li) {
    const int n = a.width[li];
    const int32_t* src = a.list[li] + row * n;
    for (int e = tid; e < n; e += UN_THREADS) {
      const int v = src[e];
      if (v >= 0 && v < a.T) atomicOr(&words[v >> 5], 1u << (v & 31));
    }
  }
  __syncthreads();
  const int per = (nwords + UN_THREADS - 1) / UN_THREADS;
  const int w0 = tid * per, w1 = min(w0 + per, nwords);
  int mine = 0;
  for (int i = w0; i < w1; ++i) mine += __popc(words[i]);
  const int incl = wave_incl_scan(mine);
  if (l == WAVE - 1) wsum[wv] = incl;
  __syncthreads();
  int off = incl - mine, total = 0;
  for (int j = 0; j < NW; ++j) {
    off += j < wv ? wsum[j] : 0;
    total += wsum[j];
  }
  int32_t* out = a.out_idx + row * a.cap;
  for (int i = w0; i < w1 && off < a.cap; ++i) {
    uint32_t m = words[i];
    while (m && off < a.cap) {
      const int bit = __ffs(m) - 1;
      out[off++] = i * 32 + bit;
      m &= m - 1;
    }
  }
  for (int e = min(total, a.cap) + tid; e < a.cap; e += UN_THREADS) out[e] = -1;
  if (tid == 0 && a.out_count) a.out_count[row] = total;
}

// ============================================================ projections
//
// The producers of the indexer's inputs are linear maps over bf16 operands:
// the query's low-rank up-projection (r = 2048 -> H*D), the head weights, and
// the m:1 key compression (the m token vectors of a group side by side).  All
// are y = x . w^T with x [M][K], w [N][K] row-major, on MFMA with fp32
// accumulation; the output goes straight to the layout the indexer reads (q
// head-major [.., H, D] bf16, w fp32), so no conversion pass follows.
//
// A workgroup computes a BM x BN tile of y over K in steps of PJ_BK = 64.
// The x and w tiles go straight from memory into LDS (global_load_lds_dwordx4:
// no staging registers, no LDS store instructions), into one of two buffers:
// the next step's tiles are requested before this step's MFMAs and waited
// for (vmcnt) before the step's barrier.  LDS rows are 128 bytes (8 pieces of
// 16 bytes); piece p of row r sits in slot p ^ ((r >> 1) & 7), so that the
// operand reads (32 rows at one piece) cover all 16 16-byte bank groups of
// each 256-byte window.  A wave fills 1-KB blocks of 8 rows, lane i writing
// row i / 8, slot i % 8, so it fetches the piece that slot holds.  Wave
// (wm, wn) owns a (32*TM) x (32*TN) sub-tile; for each 16-deep slice it reads
// TM A and TN B operands (lane: row l & 31, k half l >> 5) and issues TM*TN
// v_mfma_f32_32x32x16_bf16.  Rows past M and columns past N load a clamped
// (valid) row and are not stored.
template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * WAVE, 512 / (WGM * WGN * WAVE)) void project_kernel(ProjArgs a) {
  constexpr int NT = WGM * WGN * WAVE, NW = NT / WAVE;
  constexpr int TM = BM / WGM / 32, TN = BN / WGN / 32;
  constexpr int AC = BM / 8 / NW, BC = BN / 8 / NW;    // 1-KB blocks per wave and step
  static_assert(AC * NW * 8 == BM && BC * NW * 8 == BN && TM >= 1 && TN >= 1, "tile shape");
  __shared__ __attribute__((aligned(1024))) bf16x8 As[2][BM * 8];
  __shared__ __attribute__((aligned(1024))) bf16x8 Bs[2][BN * 8];
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int wm = wv / WGN, wn = wv % WGN;
  const long long m0 = (long long)blockIdx.x * BM;
  const int n0 = blockIdx.y * BN;
  const long long kp = a.K / 8;
  const int nk = a.K / PJ_BK;
  auto slot = [](int r, int p) { return r * 8 + (p ^ ((r >> 1) & 7)); };
  const bf16x8* asrc[AC];
  const bf16x8* bsrc[BC];
#pragma unroll
  for (int c = 0; c < AC; ++c) {
    const int r = 8 * (wv + NW * c) + (l >> 3);
    const long long gr = m0 + r < a.M ? m0 + r : a.M - 1;
    asrc[c] = (const bf16x8*)a.x + gr * kp + ((l & 7) ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const int r = 8 * (wv + NW * c) + (l >> 3);
    const long long gn = n0 + r < a.N ? n0 + r : a.N - 1;
    bsrc[c] = (const bf16x8*)a.w + gn * kp + ((l & 7) ^ ((r >> 1) & 7));
  }
  auto issue = [&](int kt, int buf) {
#pragma unroll
    for (int c = 0; c < AC; ++c) dma16(asrc[c] + kt * 8, lds_addr(&As[buf][64 * (wv + NW * c)]));
#pragma unroll
    for (int c = 0; c < BC; ++c) dma16(bsrc[c] + kt * 8, lds_addr(&Bs[buf][64 * (wv + NW * c)]));
  };
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  issue(0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue(kt + 1, cur ^ 1);
#pragma unroll
    for (int kk = 0; kk < PJ_BK / 16; ++kk) {
      const int p = 2 * kk + (l >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = As[cur][slot(wm * TM * 32 + i * 32 + (l & 31), p)];
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = Bs[cur][slot(wn * TN * 32 + j * 32 + (l & 31), p)];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c = n0 + wn * TN * 32 + j * 32 + (l & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const long long r = m0 + wm * TM * 32 + i * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
        if (r < a.M && c < a.N) {
          if (a.out_f32) ((float*)a.y)[r * a.N + c] = acc[i][j][e];
          else ((__bf16*)a.y)[r * a.N + c] = (__bf16)acc[i][j][e];
        }
      }
    }
}

// ============================================================ row sort
//
// Sorts each row of `len` (index, score) pairs by (score desc, index asc);
// -1 entries go last.  One workgroup per row, bitonic sort in LDS.

constexpr int SORT_THREADS = 256;
constexpr int SORT_MAX = 4096;

__global__ __launch_bounds__(SORT_THREADS) void sort_rows_kernel(int32_t* idx, float* score, int len) {
  __shared__ u64 keys[SORT_MAX];
  const int tid = threadIdx.x;
  int32_t* ri = idx + (size_t)blockIdx.x * len;
  float* rs = score + (size_t)blockIdx.x * len;
  int n2 = 1;
  while (n2 < len) n2 <<= 1;
  for (int e = tid; e < n2; e += SORT_THREADS) {
    u64 x = 0ull;
    if (e < len && ri[e] >= 0) x = make_key(rs[e], (uint32_t)ri[e]);
    keys[e] = x;
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int e = tid; e < n2 / 2; e += SORT_THREADS) {
        const int lo = 2 * e - (e & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;          // descending runs first -> overall descending
        const u64 x = keys[lo], y = keys[hi];
        if ((x < y) == desc) {
          keys[lo] = y;
          keys[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < len; e += SORT_THREADS) {
    const u64 x = keys[e];
    ri[e] = x ? key_index(x) : -1;
    rs[e] = x ? key_score(x) : -__builtin_inff();
  }
}

// ============================================================ set recall

constexpr int RECALL_THREADS = 256;
constexpr int RECALL_MAX_REF = 8192;

__global__ __launch_bounds__(RECALL_THREADS) void recall_kernel(const int32_t* sel, int n_sel,
                                                                const int32_t* ref, int n_ref, int T,
                                                                float* out) {
  __shared__ int32_t rs[RECALL_MAX_REF];
  __shared__ uint8_t hit[RECALL_MAX_REF];
  __shared__ int tot[2];
  const int tid = threadIdx.x;
  const int32_t* rr = ref + (size_t)blockIdx.x * n_ref;
  const int32_t* sr = sel + (size_t)blockIdx.x * n_sel;
  int n2 = 1;
  while (n2 < n_ref) n2 <<= 1;
  const int32_t BIG = 0x7FFFFFFF;
  for (int e = tid; e < n2; e += RECALL_THREADS) {
    int32_t v = BIG;
    if (e < n_ref) {
      v = rr[e];
      if (v < 0 || v >= T) v = BIG;
    }
    rs[e] = v;
    hit[e] = 0;
  }
  if (tid < 2) tot[tid] = 0;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {       // ascending bitonic sort
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int e = tid; e < n2 / 2; e += RECALL_THREADS) {
        const int lo = 2 * e - (e & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int32_t x = rs[lo], y = rs[hi];
        if ((x > y) == asc) {
          rs[lo] = y;
          rs[hi] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int e = tid; e < n_sel; e += RECALL_THREADS) {
    const int32_t v = sr[e];
    if (v < 0 || v >= T) continue;
    int lo = 0, hi = n2;                              // first position with rs[pos] >= v
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rs[mid] < v) lo = mid + 1; else hi = mid;
    }
    if (lo < n2 && rs[lo] == v) hit[lo] = 1;
  }
  __syncthreads();
  int uniq = 0, found = 0;
  for (int e = tid; e < n2; e += RECALL_THREADS) {
    const bool first = rs[e] != BIG && (e == 0 || rs[e - 1] != rs[e]);
    uniq += first;
    found += first && hit[e];
  }
  uniq = wave_sum_i32(uniq);
  found = wave_sum_i32(found);
  if ((tid & (WAVE - 1)) == 0) {
    atomicAdd(&tot[0], uniq);
    atomicAdd(&tot[1], found);
  }
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = tot[0] ? (float)tot[1] / (float)tot[0] : 1.0f;
}

// ============================================================ launchers

template <int MODE>
static const void* prefill_kernel_ptr(bool mfma, bool bf16) {
  if (mfma) return (const void*)prefill_mfma2_kernel<MODE>;
  if (bf16) return (const void*)prefill_generic_kernel<MODE, __bf16>;
  return (const void*)prefill_generic_kernel<MODE, float>;
}

static const void* prefill_kernel_for(int mode, bool mfma, bool bf16) {
  switch (mode) {
    case MODE_TOPK: return prefill_kernel_ptr<MODE_TOPK>(mfma, bf16);
    case MODE_THRESHOLD: return prefill_kernel_ptr<MODE_THRESHOLD>(mfma, bf16);
    default: return prefill_kernel_ptr<MODE_INTERLEAVED>(mfma, bf16);
  }
}

static int blocks_per_cu(const void* fn, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

int prefill_blocks_per_cu(int mode, bool mfma, bool bf16) {
  return blocks_per_cu(prefill_kernel_for(mode, mfma, bf16), mfma ? PF2_THREADS : PF_THREADS);
}

template <int MODE>
static void launch_prefill_mode(const PrefillArgs& a, bool mfma, int grid, hipStream_t st) {
  if (mfma)
    prefill_mfma2_kernel<MODE><<<grid, PF2_THREADS, 0, st>>>(a);
  else if (a.bf16)
    prefill_generic_kernel<MODE, __bf16><<<grid, PF_THREADS, 0, st>>>(a);
  else
    prefill_generic_kernel<MODE, float><<<grid, PF_THREADS, 0, st>>>(a);
}

hipError_t launch_prefill(const PrefillArgs& a, int mode, bool mfma, int grid, hipStream_t st) {
  switch (mode) {
    case MODE_TOPK: launch_prefill_mode<MODE_TOPK>(a, mfma, grid, st); break;
    case MODE_THRESHOLD: launch_prefill_mode<MODE_THRESHOLD>(a, mfma, grid, st); break;
    default: launch_prefill_mode<MODE_INTERLEAVED>(a, mfma, grid, st); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_batch(const DecodeBatch& bt, int nsplit, hipStream_t st) {
  const DecodeArgs& a = bt.a[0];
  const dim3 g1(nsplit, a.B * a.S_q, bt.L);
  if (a.chunk == DEC_CHUNK_LONG) decode_score_batch_kernel<DEC_CHUNK_LONG><<<g1, DEC_THREADS, 0, st>>>(bt);
  else decode_score_batch_kernel<DEC_CHUNK><<<g1, DEC_THREADS, 0, st>>>(bt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_select_batch_kernel<<<dim3(a.B * a.S_q, 1, bt.L), DEC_SEL_THREADS, 0, st>>>(bt);
  return hipGetLastError();
}

// Fixed device scratch for csa_index_topk_decode_noalloc: callers that
// cannot allocate get the decode workspace from this file-scope array (one
// copy per GPU, held until the process ends).  Host code never uses the
// array's name as an address: each device's address is asked once from the
// runtime and kept.
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[NOALLOC_MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int nsplit, hipStream_t st) {
  dim3 g1(nsplit, a.B * a.S_q);
  if (a.chunk == DEC_CHUNK_LONG) decode_score_kernel<DEC_CHUNK_LONG><<<g1, DEC_THREADS, 0, st>>>(a);
  else decode_score_kernel<DEC_CHUNK><<<g1, DEC_THREADS, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_select_kernel<<<a.B * a.S_q, DEC_SEL_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.S_q;
  if (rows <= 0) return hipSuccess;
  attn_chunk_kernel<<<dim3(a.nsplit, (unsigned)rows), AT_THREADS, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3(AT_H, (unsigned)rows), AT_D, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_union(const UnionArgs& a, long long rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  union_rows_kernel<<<(unsigned)rows, UN_THREADS, 0, st>>>(a);
  return hipGetLastError();
}

// variant 0: 256 x 256 tiles, 8 waves of 128 x 64; variant 1: 128 x 128 tiles,
// 4 waves of 64 x 64 (for outputs narrower than 256 columns).
long long project_rows_limit() { return (1ll << 32) / 512 * 256 - 256; }

hipError_t launch_project(const ProjArgs& a, int variant, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (variant == 0) {
    const dim3 grid((unsigned)((a.M + 255) / 256), (unsigned)((a.N + 255) / 256));
    project_kernel<256, 256, 2, 4><<<grid, 512, 0, st>>>(a);
  } else {
    const dim3 grid((unsigned)((a.M + 127) / 128), (unsigned)((a.N + 127) / 128));
    project_kernel<128, 128, 2, 2><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_sort_rows(int32_t* idx, float* score, long long rows, int len, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  sort_rows_kernel<<<(unsigned)rows, SORT_THREADS, 0, st>>>(idx, score, len);
  return hipGetLastError();
}

hipError_t launch_recall(const int32_t* sel, int n_sel, const int32_t* ref, int n_ref, long long rows,
                         int T, float* out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  recall_kernel<<<(unsigned)rows, RECALL_THREADS, 0, st>>>(sel, n_sel, ref, n_ref, T, out);
  return hipGetLastError();
}

}  // namespace csa
