// HIP kernels (gfx950) for the CSA lightning-indexer top-k step.
//
// Score (per query t, key s):  I = sum_j w[t,j] * max(q[t,j] . k[s], 0).
// Every kernel streams key tiles, forms scores in registers and feeds a
// per-query running top-k; the [B,S,H,T] score tensor is never formed.
//
// Prefill family (top-k, threshold, interleaved partitions):
//   persistent grid; a workgroup owns PF_ROWS = 8 consecutive query rows, a
//   wave owns 2 of them ("slots": lanes 0-31 -> slot 0, lanes 32-63 -> slot 1).
//   Per key tile the wave produces one score per lane, filters it against the
//   slot's running threshold key and appends survivors to the slot's candidate
//   buffer in the workspace.  A full buffer is compacted to the exact top-k
//   (radix select), which raises the threshold; at the end the exact top-k of
//   the buffer is emitted.
// Decode: scores of a few queries against a long key range, split across
//   many workgroups (HBM-bound), then one workgroup per row selects.
#include "csa_device.hpp"
#include "csa_internal.hpp"

namespace csa {

// ============================================================ shared pieces

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

// Wave-uniform top-k state of a wave's two query slots.
struct SlotPair {
  u64* cand[2];
  int cnt[2];
  u64 thr[2];     // keys below thr[s] cannot enter slot s's top-k
  int surv[2];    // threshold mode: keys >= thr_fixed seen
};

// Keep the exact top-kk of buf[0..cnt) in place; returns the new threshold.
__device__ u64 wave_compact(u64* buf, int cnt, int kk, uint32_t* hist) {
  const int l = lane_id();
  const u64 T = wave_select_kth(buf, cnt, kk, hist);
  int w = 0;
  for (int base = 0; base < cnt; base += WAVE) {
    const int i = base + l;
    const u64 x = i < cnt ? buf[i] : 0ull;
    const bool keep = i < cnt && x >= T;
    const u64 m = ballot(keep);
    if (keep) buf[w + lanes_below(m)] = x;   // w + rank <= i: never ahead of the reads
    w += __popcll(m);
  }
  return T + 1ull;
}

template <int MODE>
__device__ __forceinline__ void wave_offer(SlotPair& st, u64 key, bool valid, const PrefillArgs& a,
                                           uint32_t* hist) {
  const int l = lane_id();
  const int slot = l >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    if (st.cnt[s] + 32 > a.C) {                       // make room: at most 32 appends per slot
      u64 t = wave_compact(st.cand[s], st.cnt[s], a.kk, hist);
      st.thr[s] = t > st.thr[s] ? t : st.thr[s];
      st.cnt[s] = a.kk;
    }
  }
  if (MODE == MODE_THRESHOLD) {
    const u64 ms = ballot(valid && key >= a.thr_fixed);
    st.surv[0] += __popc((uint32_t)ms);
    st.surv[1] += __popc((uint32_t)(ms >> 32));
  }
  const u64 thr = slot ? st.thr[1] : st.thr[0];
  const bool keep = valid && key >= thr;
  const u64 m = ballot(keep);
  const int n0 = __popc((uint32_t)m), n1 = __popc((uint32_t)(m >> 32));
  if (keep) {
    const int pos = lanes_below(m) - (slot ? n0 : 0);
    u64* dst = slot ? st.cand[1] : st.cand[0];
    dst[(slot ? st.cnt[1] : st.cnt[0]) + pos] = key;
  }
  st.cnt[0] += n0;
  st.cnt[1] += n1;
}

// Emit the exact top-kk of buf[0..cnt) (all of it when cnt <= kk) to one
// output row of kk entries, then pad with -1 / -inf.
__device__ void wave_emit(const u64* buf, int cnt, int kk, uint32_t* hist, int32_t* oi, float* os) {
  const int l = lane_id();
  u64 T = 0ull;
  if (cnt > kk) T = wave_select_kth(buf, cnt, kk, hist);
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
  int w = 0;
  for (int base = 0; base < cnt; base += WAVE) {
    const int i = base + l;
    const u64 x = i < cnt ? buf[i] : 0ull;
    const bool keep = i < cnt && x >= T;
    const u64 m = ballot(keep);
    const int pos = w + lanes_below(m);
    if (keep && pos < kk) {                           // exactly kk pass; the bound only guards the row
      oi[pos] = key_index(x);
      if (os) os[pos] = key_score(x);
    }
    w += __popcll(m);
  }
  w = w < kk ? w : kk;
  for (int i = w + l; i < kk; i += WAVE) {
    oi[i] = -1;
    if (os) os[i] = -__builtin_inff();
  }
}

// Rows whose visible keys all fit (vis <= kk) and whose scores are not asked
// for: the selection is every visible key.
__device__ void wave_emit_all_visible(int vis, int part, int P, int kk, int32_t* oi) {
  const int l = lane_id();
  for (int i = l; i < kk; i += WAVE) oi[i] = i < vis ? part + P * i : -1;
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

template <int MODE>
__device__ void finish_rows(const PrefillArgs& a, SlotPair& st, int b, int r0, int part,
                            uint32_t* hist) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int row = r0 + s;
    if (row >= a.S_q) continue;
    const size_t orow = (size_t)b * a.S_q + row;
    int32_t* oi = a.out_idx + orow * a.out_stride + (size_t)part * a.kk;
    float* os = a.out_score ? a.out_score + orow * a.out_stride + (size_t)part * a.kk : nullptr;
    wave_emit(st.cand[s], st.cnt[s], a.kk, hist, oi, os);
    if (MODE == MODE_THRESHOLD && lane_id() == 0) a.out_count[orow] = st.surv[s];
  }
}

template <int MODE>
__device__ __forceinline__ bool block_needs_scores(const PrefillArgs& a, int b, int qb, int part,
                                                   int& vis_max) {
  vis_max = 0;
  bool need = MODE == MODE_THRESHOLD || a.need_scores;
  for (int r = 0; r < PF_ROWS; ++r) {
    const int v = row_visible(a, b, qb * PF_ROWS + r, part);
    vis_max = v > vis_max ? v : vis_max;
    need = need || v > a.kk;
  }
  return need;
}

// ============================================================ MFMA prefill
//
// bf16, H = 64 heads, D = 128.  One wave multiplies its 2 queries x 64 heads
// (4 row tiles of 32 heads, held as MFMA A operands in registers) with 32-key
// column tiles read from LDS: v_mfma_f32_32x32x16_bf16, fp32 accumulation,
// 8 steps over D.  Output lane l holds key column (l & 31) and 16 heads of a
// row tile; ReLU and the head weights are applied in registers, the two lane
// halves are summed, and each lane ends with one (slot, key) score.

constexpr int MH = 64, MD = 128;
constexpr int KROW = MD + 8;   // LDS row pitch in bf16 (272 B): conflict-free 16-B reads

template <int MODE>
__global__ __launch_bounds__(PF_THREADS) void prefill_mfma_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) __bf16 ktile[2][PF_KTILE * KROW];
  __shared__ float wsh[PF_ROWS][MH];
  __shared__ uint32_t hist_all[PF_THREADS / WAVE][SEL_BINS];

  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  uint32_t* hist = hist_all[wv];
  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;

  for (int r = 0;; ++r) {
    const int it = round_item(r);
    if (r * (int)gridDim.x >= a.n_items) break;
    if (it >= a.n_items) continue;
    int b, qb, part;
    decode_item(a, it, b, qb, part);
    int vis_max;
    const bool need = block_needs_scores<MODE>(a, b, qb, part, vis_max);
    const int r0 = qb * PF_ROWS + 2 * wv;             // this wave's two rows
    const int vis0 = row_visible(a, b, r0, part), vis1 = row_visible(a, b, r0 + 1, part);
    if (!need) {
      for (int s = 0; s < 2; ++s) {
        const int row = r0 + s;
        if (row >= a.S_q) continue;
        const size_t orow = (size_t)b * a.S_q + row;
        wave_emit_all_visible(s ? vis1 : vis0, part, a.P, a.kk,
                              a.out_idx + orow * a.out_stride + (size_t)part * a.kk);
      }
      continue;
    }

    __syncthreads();                                  // LDS of the previous item is free
    for (int e = tid; e < PF_ROWS * MH; e += PF_THREADS) {
      const int rr = e / MH, h = e % MH, row = qb * PF_ROWS + rr;
      wsh[rr][h] = row < a.S_q ? a.w[((size_t)b * a.S_q + row) * MH + h] : 0.f;
    }
    bf16x8 A[4][8];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int row = r0 + (rt >> 1);
      if (row < a.S_q) {
        const bf16x8* src = (const bf16x8*)(Q + (((size_t)b * a.S_q + row) * MH + (rt & 1) * 32 + (l & 31)) * MD);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) A[rt][kk] = src[2 * kk + (l >> 5)];
      } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) A[rt][kk] = bf16x8{};
      }
    }
    SlotPair st;
    st.cand[0] = a.cand + ((size_t)blockIdx.x * PF_ROWS + 2 * wv) * a.C;
    st.cand[1] = st.cand[0] + a.C;
    st.cnt[0] = st.cnt[1] = 0;
    st.thr[0] = st.thr[1] = (MODE == MODE_THRESHOLD) ? a.thr_fixed : 0ull;
    st.surv[0] = st.surv[1] = 0;

    const int ntiles = (vis_max + PF_KTILE - 1) / PF_KTILE;
    // stage loader: 64 rows x 16 chunks of 16 B; 4 chunks per thread
    u32x4 stage[4];
    auto load_tile = [&](int t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = tid + e * PF_THREADS, row = c >> 4, col = c & 15;
        const int j = t * PF_KTILE + row;
        if (j < vis_max) {
          const size_t s = (size_t)part + (size_t)a.P * j;
          stage[e] = *(const u32x4*)(K + ((size_t)b * a.T + s) * MD + col * 8);
        } else {
          stage[e] = u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = tid + e * PF_THREADS, row = c >> 4, col = c & 15;
        *(u32x4*)(&ktile[buf][row * KROW + col * 8]) = stage[e];
      }
    };
    if (ntiles > 0) {
      load_tile(0);
      store_tile(0);
    }
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      if (t + 1 < ntiles) load_tile(t + 1);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x16 acc[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) acc[rt] = f32x16{};
        const __bf16* kb = &ktile[buf][(c * 32 + (l & 31)) * KROW + 8 * (l >> 5)];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8 bfr = *(const bf16x8*)(kb + 16 * kk);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][kk], bfr, acc[rt], 0, 0, 0);
        }
        float part0 = 0.f, part1 = 0.f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float* wr = &wsh[2 * wv + (rt >> 1)][(rt & 1) * 32 + 4 * (l >> 5)];
          float ps = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float x = acc[rt][i];
            ps = __builtin_fmaf(wr[8 * (i >> 2) + (i & 3)], x > 0.f ? x : 0.f, ps);
          }
          if (rt >> 1) part1 += ps; else part0 += ps;
        }
        const float o0 = __shfl_xor(part0, 32, WAVE);
        const float o1 = __shfl_xor(part1, 32, WAVE);
        const float score = (l < 32) ? part0 + o0 : part1 + o1;
        const int j = t * PF_KTILE + c * 32 + (l & 31);
        const bool valid = j < ((l < 32) ? vis0 : vis1);
        const u64 key = make_key(score, (uint32_t)(part + a.P * j));
        wave_offer<MODE>(st, key, valid, a, hist);
      }
      if (t + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    }
    finish_rows<MODE>(a, st, b, r0, part, hist);
  }
}

// ============================================================ generic prefill
//
// Any H, D and dtype (fp32 or bf16): each lane computes one (slot, key)
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
  __shared__ uint32_t hist_all[PF_THREADS / WAVE][SEL_BINS];
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  uint32_t* hist = hist_all[wv];
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
    const int r0 = qb * PF_ROWS + 2 * wv;
    const int vis0 = row_visible(a, b, r0, part), vis1 = row_visible(a, b, r0 + 1, part);
    if (!need) {
      for (int s = 0; s < 2; ++s) {
        const int row = r0 + s;
        if (row >= a.S_q) continue;
        const size_t orow = (size_t)b * a.S_q + row;
        wave_emit_all_visible(s ? vis1 : vis0, part, a.P, a.kk,
                              a.out_idx + orow * a.out_stride + (size_t)part * a.kk);
      }
      continue;
    }
    SlotPair st;
    st.cand[0] = a.cand + ((size_t)blockIdx.x * PF_ROWS + 2 * wv) * a.C;
    st.cand[1] = st.cand[0] + a.C;
    st.cnt[0] = st.cnt[1] = 0;
    st.thr[0] = st.thr[1] = (MODE == MODE_THRESHOLD) ? a.thr_fixed : 0ull;
    st.surv[0] = st.surv[1] = 0;

    const int slot = l >> 5;
    const int row = r0 + slot;
    const int vis_me = slot ? vis1 : vis0;
    const int vmax = vis0 > vis1 ? vis0 : vis1;
    const size_t qoff = ((size_t)b * a.S_q + (row < a.S_q ? row : 0)) * a.H;
    for (int j0 = 0; j0 < vmax; j0 += 32) {
      const int j = j0 + (l & 31);
      const bool valid = j < vis_me;
      float score = 0.f;
      uint32_t s_idx = 0;
      if (valid) {
        s_idx = (uint32_t)(part + a.P * j);
        const size_t koff = ((size_t)b * a.T + s_idx) * a.D;
        for (int h = 0; h < a.H; ++h) {
          float dot = 0.f;
          const size_t qh = (qoff + h) * a.D;
          for (int d = 0; d < a.D; ++d) dot = __builtin_fmaf(ld_f32(Q, qh + d), ld_f32(K, koff + d), dot);
          score = __builtin_fmaf(a.w[qoff + h], dot > 0.f ? dot : 0.f, score);
        }
      }
      wave_offer<MODE>(st, make_key(score, s_idx), valid, a, hist);
    }
    finish_rows<MODE>(a, st, b, r0, part, hist);
  }
}

// ============================================================ decode
//
// decode_score: grid (nsplit, B*S_q).  Workgroup x scans keys
// [x*chunk, (x+1)*chunk) of one query row; each wave takes 64-key steps.  The
// key rows go straight from HBM into MFMA B operands (16 B per lane); the
// query's 64x128 A operand and the lane's head weights stay in registers.

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

__global__ __launch_bounds__(DEC_THREADS) void decode_score_kernel(DecodeArgs a) {
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int row = blockIdx.y, b = row / a.S_q, i = row % a.S_q;
  const int vis = decode_visible(a, b, i);
  const int start = blockIdx.x * a.chunk;
  const int end = start + a.chunk < vis ? start + a.chunk : vis;
  if (start >= end) return;
  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;

  bf16x8 A[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const bf16x8* src = (const bf16x8*)(Q + ((size_t)row * MH + rt * 32 + (l & 31)) * MD);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) A[rt][kk] = src[2 * kk + (l >> 5)];
  }
  float wl[2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      wl[rt][e] = a.w[(size_t)row * MH + rt * 32 + 8 * (e >> 2) + 4 * (l >> 5) + (e & 3)];

  float* out = a.scores + (size_t)row * a.T;
  for (int base = start + 64 * wv; base < end; base += 64 * (DEC_THREADS / WAVE)) {
    bf16x8 Bf[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int s = base + 32 * c + (l & 31);
      s = s < end ? s : end - 1;
      const bf16x8* src = (const bf16x8*)(K + ((size_t)b * a.T + s) * MD);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) Bf[c][kk] = src[2 * kk + (l >> 5)];
    }
    float part[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[rt][kk], Bf[c][kk], acc[rt], 0, 0, 0);
      float ps = 0.f;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float x = acc[rt][e];
          ps = __builtin_fmaf(wl[rt][e], x > 0.f ? x : 0.f, ps);
        }
      part[c] = ps;
    }
    const float o0 = __shfl_xor(part[0], 32, WAVE);
    const float o1 = __shfl_xor(part[1], 32, WAVE);
    const float score = (l < 32) ? part[0] + o0 : part[1] + o1;
    const int s = base + l;                 // lanes 0-31: column tile 0, lanes 32-63: tile 1
    if (s < end) out[s] = score;
  }
}

// decode_select: one workgroup per query row; exact top-kk of the row's
// dense scores, emitted in index order of a deterministic block scan.
__global__ __launch_bounds__(DEC_SEL_THREADS) void decode_select_kernel(DecodeArgs a) {
  __shared__ uint32_t hist[SEL_BINS];
  __shared__ u64 red[2 * DEC_SEL_THREADS / WAVE];
  __shared__ int wcnt[DEC_SEL_THREADS / WAVE];
  constexpr int NW = DEC_SEL_THREADS / WAVE;
  const int tid = threadIdx.x, wv = tid / WAVE, l = tid & (WAVE - 1);
  const int row = blockIdx.x, b = row / a.S_q, i = row % a.S_q;
  const int vis = decode_visible(a, b, i);
  const float* sc = a.scores + (size_t)row * a.T;
  int32_t* oi = a.out_idx + (size_t)row * a.kk;
  float* os = a.out_score ? a.out_score + (size_t)row * a.kk : nullptr;
  u64 T = 0ull;
  if (vis > a.kk) T = block_select_kth_dense<DEC_SEL_THREADS>(sc, vis, a.kk, hist, red);
  int w = 0;
  for (int base = 0; base < vis; base += DEC_SEL_THREADS) {
    const int s = base + tid;
    u64 x = 0ull;
    bool keep = false;
    if (s < vis) {
      x = make_key(sc[s], (uint32_t)s);
      keep = x >= T;
    }
    const u64 m = ballot(keep);
    if (l == 0) wcnt[wv] = __popcll(m);
    __syncthreads();
    int off = 0, tot = 0;
    for (int j = 0; j < NW; ++j) {
      off += j < wv ? wcnt[j] : 0;
      tot += wcnt[j];
    }
    const int pos = w + off + lanes_below(m);
    if (keep && pos < a.kk) {
      oi[pos] = s;
      if (os) os[pos] = key_score(x);
    }
    w += tot;
    __syncthreads();
  }
  w = w < a.kk ? w : a.kk;
  for (int e = w + tid; e < a.kk; e += DEC_SEL_THREADS) {
    oi[e] = -1;
    if (os) os[e] = -__builtin_inff();
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
  if (mfma) return (const void*)prefill_mfma_kernel<MODE>;
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

int prefill_blocks_per_cu(int mode, bool mfma, bool bf16) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, prefill_kernel_for(mode, mfma, bf16), PF_THREADS, 0) !=
          hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

template <int MODE>
static void launch_prefill_mode(const PrefillArgs& a, bool mfma, int grid, hipStream_t st) {
  if (mfma)
    prefill_mfma_kernel<MODE><<<grid, PF_THREADS, 0, st>>>(a);
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

hipError_t launch_decode(const DecodeArgs& a, int nsplit, hipStream_t st) {
  dim3 g1(nsplit, a.B * a.S_q);
  decode_score_kernel<<<g1, DEC_THREADS, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_select_kernel<<<a.B * a.S_q, DEC_SEL_THREADS, 0, st>>>(a);
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
