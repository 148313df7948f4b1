// Device primitives for the CSA indexer kernels (gfx950, wave64).
//
// Total order.  A selection key packs (score, index) into 64 bits so that a
// larger key is a better key: the high word is the score mapped to an unsigned
// integer with the same order (sign-flip transform used by radix sorts, after
// turning -0.0 into +0.0 so that the two zeros tie), the low word is
// 0xFFFFFFFF - index so that among equal scores the lower index wins.  All
// keys are distinct, so "the k largest keys" is an exact, tie-free top-k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef unsigned long long u64;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int WAVE = 64;

// ---------------------------------------------------------------- keys

__device__ __forceinline__ uint32_t score_order_bits(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;                      // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float order_bits_score(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ u64 make_key(float s, uint32_t idx) {
  return ((u64)score_order_bits(s) << 32) | (u64)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ int key_index(u64 key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ float key_score(u64 key) { return order_bits_score((uint32_t)(key >> 32)); }

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// (the i1 form: no round trip of the predicate through a VGPR)
__device__ __forceinline__ u64 ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(u64 mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Order this wave's earlier global stores before its later global loads of
// the same addresses.  A workgroup-scope fence lowers to no wait at all here,
// and a load issued while a store to its address is still in flight can
// return the old contents; draining the vector memory counter (vmcnt = 0,
// other counters untouched) completes the stores first.
__device__ __forceinline__ void wave_own_stores_visible() {
  __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0) expcnt(7) lgkmcnt(15)
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ u64 wave_min_u64(u64 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    u64 t = __shfl_xor(v, o, WAVE);
    v = t < v ? t : v;
  }
  return v;
}

__device__ __forceinline__ u64 wave_max_u64(u64 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    u64 t = __shfl_xor(v, o, WAVE);
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, WAVE));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, WAVE));
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Inclusive prefix sum over lanes 0..63.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    int t = __shfl_up(v, o, WAVE);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int clz64(u64 x) { return __clzll((long long)x); }

// ---------------------------------------------------------------- radix select
//
// Exact k-th largest key by most-significant-digit radix refinement.  The
// digits start below the bits that all keys share (common prefix of min and
// max), RB bits per pass, histogrammed in LDS.  A pass narrows to the bin that
// holds rank k; it stops as soon as that whole bin is inside the top k, so
// the result T satisfies |{key >= T}| == k exactly.

constexpr int SEL_RB = 11;
constexpr int SEL_BINS = 1 << SEL_RB;

struct BinPick {
  int bin;    // chosen bin
  int above;  // keys in bins above it
  int count;  // keys in it
};

// Given a histogram of `nb` bins (nb <= SEL_BINS, a power of two, 16-byte
// aligned) in LDS, find the bin that holds rank `rank` counted from the top.
// Whole wave calls it; result is uniform.  Two levels: lane l sums its run of
// nb/64 bins (lane 0 the highest run) with 16-byte reads, a scan finds the run
// holding the rank, then one bin of that run per lane and a second scan find
// the bin.  Inconsistent counts (no run or bin holds the rank) give count 0.
__device__ __forceinline__ BinPick wave_pick_bin(const uint32_t* hist, int nb, int rank) {
  const int l = lane_id();
  const int per = nb >= WAVE ? nb / WAVE : 1;
  const int lo_bin = nb - (l + 1) * per;          // this lane's run: lo_bin .. lo_bin + per - 1
  int s = 0;
  if (lo_bin >= 0) {
    if ((per & 3) == 0) {
      for (int j = 0; j < per; j += 4) {
        const uint4 h = *(const uint4*)&hist[lo_bin + j];
        s += (int)(h.x + h.y + h.z + h.w);
      }
    } else {
      for (int j = 0; j < per; ++j) s += (int)hist[lo_bin + j];
    }
  }
  const int incl = wave_incl_scan(s);
  const int excl = incl - s;
  const u64 who = ballot(lo_bin >= 0 && excl < rank && rank <= incl);
  BinPick r{0, 0, 0};
  if (!who) return r;
  const int src = (int)__builtin_ctzll(who);
  const int top = nb - 1 - src * per;             // highest bin of the chosen run
  const int above = __builtin_amdgcn_readlane(excl, src);
  const int h = l < per ? (int)hist[top - l] : 0; // lane i: bin top - i
  const int incl2 = above + wave_incl_scan(h);
  const u64 hit = ballot(l < per && incl2 - h < rank && rank <= incl2);
  if (!hit) return r;
  const int s2 = (int)__builtin_ctzll(hit);
  r.bin = top - s2;
  r.count = __builtin_amdgcn_readlane(h, s2);
  r.above = __builtin_amdgcn_readlane(incl2, s2) - r.count;
  return r;
}

// Zero hist[0..nb) (16-byte aligned) with 16-byte stores where nb allows.
__device__ __forceinline__ void wave_clear_hist(uint32_t* hist, int nb) {
  const int l = lane_id();
  if (nb >= 4 * WAVE) {
    for (int b = 4 * l; b < nb; b += 4 * WAVE) *(uint4*)&hist[b] = make_uint4(0u, 0u, 0u, 0u);
  } else {
    for (int b = l; b < nb; b += WAVE) hist[b] = 0u;
  }
}

// The r-th largest of w distinct keys list[0..w) (1 <= r <= w <= WAVE): the
// key with exactly r - 1 keys above it, found by comparing every pair (each
// lane holds one key and compares it with all others via readlane).
__device__ __forceinline__ u64 wave_small_kth(const u64* list, int w, int r) {
  const int l = lane_id();
  const u64 v = l < w ? list[l] : 0ull;
  const uint32_t vh = (uint32_t)(v >> 32), vl = (uint32_t)v;
  int g = 0;
  for (int s = 0; s < w; ++s) {
    const u64 o = ((u64)(uint32_t)__builtin_amdgcn_readlane((int)vh, s) << 32) |
                  (uint32_t)__builtin_amdgcn_readlane((int)vl, s);
    g += o > v ? 1 : 0;
  }
  const u64 m = ballot(l < w && g == r - 1);
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  return ((u64)(uint32_t)__builtin_amdgcn_readlane((int)vh, src) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)vl, src);
}

// ---------------------------------------------------------------- register-resident select
//
// The same refinement over keys held in registers: x[j] is the key of element
// j*WAVE + lane (wave version) or j*NT + tid (block version), 0 for empty
// slots (0 is below every real key: its score word would have to be a NaN).
// Keys are loaded once with all loads in flight; each pass only reads
// registers and LDS.

__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, WAVE));
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Linear score bins between the smallest and largest score of a key set.
// Monotone in the score (IEEE subtraction, multiplication, the truncating
// conversion and the integer clamp never reverse an order), so every key in a higher
// bin beats every key in a lower one: the bin holding rank k is the only one
// that needs exact resolution.  Scores of typical rows share a few exponents,
// which would crowd a first radix digit on raw bits into a handful of bins.
struct LinBins {
  float lo, scale;
  // (key_score(key) - lo) * scale >= 0 for every key of the set: truncate,
  // then clamp the top bin as an integer (no float min and its canonicalize)
  __device__ __forceinline__ int operator()(u64 key) const {
    const uint32_t b = (uint32_t)((key_score(key) - lo) * scale);
    return (int)(b < (uint32_t)(SEL_BINS - 1) ? b : (uint32_t)(SEL_BINS - 1));
  }
};

__device__ __forceinline__ bool lin_bins_ok(float lo, float hi, LinBins& lb) {
  const float range = hi - lo;
  lb.lo = lo;
  lb.scale = (float)SEL_BINS / range;
  return range > 0.f && lb.scale > 0.f && lb.scale < __builtin_inff();
}

constexpr int WAVE_LIST = 256;    // keys of one linear bin resolved by a wave from LDS

struct AnyKey {
  __device__ __forceinline__ bool operator()(u64 v) const { return v != 0ull; }
};
struct InBin {
  LinBins lb;
  int bin;
  __device__ __forceinline__ bool operator()(u64 v) const { return v != 0ull && lb(v) == bin; }
};

// Exact k-th largest of the keys accepted by `in` (more than k of them) by
// most-significant-digit radix refinement from registers.  key(j) returns
// the key of element j*WAVE + lane (0 = empty), for j < R with j*WAVE < n; it
// is recomputed on every pass, so a caller may keep its keys in any compact
// form.
// A uniform bound re-read at the start of a pass: the compiler then compares
// slot indices against it afresh in each pass instead of keeping one
// 64-bit condition per slot alive across passes (which spills).
// (n is the same in every lane.)
__device__ __forceinline__ int fresh_bound(int n) {
  n = __builtin_amdgcn_readfirstlane(n);
  asm volatile("" : "+s"(n));
  return n;
}

template <int R, typename KeyAt, typename Pred>
__device__ __forceinline__ u64 wave_radix_kth_at(KeyAt key, int n, int k, uint32_t* hist, Pred in) {
  u64 lo = ~0ull, hi = 0ull;
  key.fresh();
  int nn = fresh_bound(n);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j * WAVE < nn) {
      const u64 v = key(j);
      if (in(v)) {
        lo = v < lo ? v : lo;
        hi = v > hi ? v : hi;
      }
    }
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (lo == hi) return lo;
  int hi_bit = 64 - clz64(lo ^ hi);
  u64 prefix = hi_bit >= 64 ? 0ull : (lo >> hi_bit);
  int rank = k;
  while (true) {
    const int rb = hi_bit < SEL_RB ? hi_bit : SEL_RB;
    const int shift = hi_bit - rb;
    const int nb = 1 << rb;
    const uint32_t dmask = (uint32_t)(nb - 1);
    wave_clear_hist(hist, nb);
    wave_lds_sync();
    key.fresh();
    nn = fresh_bound(n);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (j * WAVE < nn) {
        const u64 v = key(j);
        const bool match = in(v) && (hi_bit >= 64 || (v >> hi_bit) == prefix);
        if (match) atomicAdd(&hist[(uint32_t)(v >> shift) & dmask], 1u);
      }
    }
    wave_lds_sync();
    const BinPick pk = wave_pick_bin(hist, nb, rank);
    wave_lds_sync();
    rank -= pk.above;
    prefix = (prefix << rb) | (u64)pk.bin;
    hi_bit = shift;
    if (pk.count == rank || shift == 0) return prefix << shift;
  }
}

// Key accessors for the register selects.  fresh() runs at the start of
// every pass over the keys: an accessor that derives keys from a compact form
// launders its base there, so that the compiler recomputes the per-slot
// values in each pass instead of keeping all of them live across passes.
template <int R>
struct ArrayKeys {
  const u64 (&x)[R];
  __device__ __forceinline__ u64 operator()(int j) const { return x[j]; }
  __device__ __forceinline__ void fresh() {}
};

// The same over keys held as an array.
template <int R, typename Pred>
__device__ __forceinline__ u64 wave_radix_kth(const u64 (&x)[R], int n, int k, uint32_t* hist, Pred in) {
  return wave_radix_kth_at<R>(ArrayKeys<R>{x}, n, k, hist, in);
}

// The r-th largest of w distinct keys list[0..w) (1 <= r <= w <= WAVE_LIST).
__device__ __forceinline__ u64 wave_list_kth(const u64* list, int w, int r, uint32_t* hist) {
  const int l = lane_id();
  if (w <= WAVE) return wave_small_kth(list, w, r);
  constexpr int RL = WAVE_LIST / WAVE;
  u64 y[RL];
#pragma unroll
  for (int j = 0; j < RL; ++j) {
    const int i = j * WAVE + l;
    y[j] = i < w ? list[i] : 0ull;
  }
  wave_lds_sync();
  return wave_radix_kth(y, w, r, hist, AnyKey{});
}

// ---------------------------------------------------------------- streaming select
//
// The same selection over keys in global memory written earlier by this
// wave (its candidate buffer), for use while the wave's MFMA operands occupy
// the registers: every pass streams the buffer with 8 loads in flight per lane.

constexpr int STREAM_BATCH = 16;

template <typename F>
__device__ __forceinline__ void wave_stream(const u64* buf, int n, F f) {
  const int l = lane_id();
  for (int base = 0; base < n; base += STREAM_BATCH * WAVE) {
    // Unconditional loads from clamped addresses, so that the whole batch is in
    // flight at once (a load under an i < n branch is waited on by itself);
    // candidate buffers stream past L2.
    u64 v[STREAM_BATCH];
#pragma unroll
    for (int j = 0; j < STREAM_BATCH; ++j) {
      const int i = base + j * WAVE + l;
      v[j] = __builtin_nontemporal_load(&buf[i < n ? i : n - 1]);
    }
#pragma unroll
    for (int j = 0; j < STREAM_BATCH; ++j)
      if (base + j * WAVE + l >= n) v[j] = 0ull;
#pragma unroll
    for (int j = 0; j < STREAM_BATCH; ++j) f(v[j], base + j * WAVE);   // 0 = past the end
  }
}

template <typename Pred>
__device__ __forceinline__ u64 wave_radix_kth_stream(const u64* buf, int n, int k, uint32_t* hist, Pred in) {
  const int l = lane_id();
  u64 lo = ~0ull, hi = 0ull;
  wave_stream(buf, n, [&](u64 v, int) {
    if (in(v)) {
      lo = v < lo ? v : lo;
      hi = v > hi ? v : hi;
    }
  });
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (lo == hi) return lo;
  int hi_bit = 64 - clz64(lo ^ hi);
  u64 prefix = hi_bit >= 64 ? 0ull : (lo >> hi_bit);
  int rank = k;
  while (true) {
    const int rb = hi_bit < SEL_RB ? hi_bit : SEL_RB;
    const int shift = hi_bit - rb;
    const int nb = 1 << rb;
    const uint32_t dmask = (uint32_t)(nb - 1);
    wave_clear_hist(hist, nb);
    wave_lds_sync();
    wave_stream(buf, n, [&](u64 v, int) {
      if (in(v) && (hi_bit >= 64 || (v >> hi_bit) == prefix)) atomicAdd(&hist[(uint32_t)(v >> shift) & dmask], 1u);
    });
    wave_lds_sync();
    const BinPick pk = wave_pick_bin(hist, nb, rank);
    wave_lds_sync();
    rank -= pk.above;
    prefix = (prefix << rb) | (u64)pk.bin;
    hi_bit = shift;
    if (pk.count == rank || shift == 0) return prefix << shift;
  }
}

// Exact k-th largest key of buf[0..n) (n > k >= 1): linear-bin histogram,
// gather of the bin holding rank k into `list`, radix resolution.  slo/shi
// are per-lane bounds on the scores in the buffer (the caller tracked them
// while appending; +inf/-inf where a lane saw none).
__device__ __forceinline__ u64 wave_select_kth_stream(const u64* buf, int n, int k, uint32_t* hist, u64* list,
                                                      float slo, float shi) {
  const int l = lane_id();
  wave_own_stores_visible();
  slo = wave_min_f32(slo);
  shi = wave_max_f32(shi);
  LinBins lb;
  if (!lin_bins_ok(slo, shi, lb)) return wave_radix_kth_stream(buf, n, k, hist, AnyKey{});
  wave_clear_hist(hist, SEL_BINS);
  wave_lds_sync();
  wave_stream(buf, n, [&](u64 v, int) {
    if (v) atomicAdd(&hist[lb(v)], 1u);
  });
  wave_lds_sync();
  const BinPick pk = wave_pick_bin(hist, SEL_BINS, k);
  wave_lds_sync();
  const int r = k - pk.above;
  const InBin inb{lb, pk.bin};
  if (pk.count > WAVE_LIST) return wave_radix_kth_stream(buf, n, r, hist, inb);
  int w = 0;
  wave_stream(buf, n, [&](u64 v, int) {
    const bool in = inb(v);
    const u64 m = ballot(in);
    if (in) list[w + lanes_below(m)] = v;
    w += __popcll(m);
  });
  wave_lds_sync();
  if (w <= WAVE) return wave_small_kth(list, w, r);
  constexpr int RL = WAVE_LIST / WAVE;
  u64 y[RL];
#pragma unroll
  for (int j = 0; j < RL; ++j) {
    const int i = j * WAVE + l;
    y[j] = i < w ? list[i] : 0ull;
  }
  wave_lds_sync();
  if (w == r) {
    u64 mn = ~0ull;
#pragma unroll
    for (int j = 0; j < RL; ++j) mn = (y[j] && y[j] < mn) ? y[j] : mn;
    return wave_min_u64(mn);
  }
  return wave_radix_kth(y, w, r, hist, AnyKey{});
}

// Block-level select over dense fp32 scores in global memory (implicit
// indices idx = i), for rows too long for registers.  Requires n > k >= 1.
template <int NT>
__device__ __forceinline__ u64 block_select_kth_dense(const float* sc, int n, int k, uint32_t* hist, u64* red) {
  const int tid = threadIdx.x;
  const int l = lane_id(), wv = tid / WAVE;
  constexpr int NW = NT / WAVE;
  u64 lo = ~0ull, hi = 0ull;
#pragma unroll 8
  for (int i = tid; i < n; i += NT) {
    const u64 x = make_key(sc[i], (uint32_t)i);
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  }
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  if (l == 0) { red[wv] = lo; red[NW + wv] = hi; }
  __syncthreads();
  lo = ~0ull; hi = 0ull;
  for (int j = 0; j < NW; ++j) {
    lo = red[j] < lo ? red[j] : lo;
    hi = red[NW + j] > hi ? red[NW + j] : hi;
  }
  __syncthreads();
  if (lo == hi) return lo;
  int hi_bit = 64 - clz64(lo ^ hi);
  u64 prefix = hi_bit >= 64 ? 0ull : (lo >> hi_bit);
  int rank = k;
  while (true) {
    const int rb = hi_bit < SEL_RB ? hi_bit : SEL_RB;
    const int shift = hi_bit - rb;
    const int nb = 1 << rb;
    const uint32_t dmask = (uint32_t)(nb - 1);
    for (int b = tid; b < nb; b += NT) hist[b] = 0u;
    __syncthreads();
#pragma unroll 8
    for (int i = tid; i < n; i += NT) {
      const u64 x = make_key(sc[i], (uint32_t)i);
      const bool match = hi_bit >= 64 || (x >> hi_bit) == prefix;
      if (match) atomicAdd(&hist[(uint32_t)(x >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      const BinPick pk = wave_pick_bin(hist, nb, rank);
      if (l == 0) { red[0] = (u64)pk.bin; red[1] = (u64)pk.above; red[2] = (u64)pk.count; }
    }
    __syncthreads();
    const int bin = (int)red[0], above = (int)red[1], cnt = (int)red[2];
    __syncthreads();
    rank -= above;
    prefix = (prefix << rb) | (u64)bin;
    hi_bit = shift;
    if (cnt == rank || shift == 0) return prefix << shift;
  }
}

}  // namespace csa
