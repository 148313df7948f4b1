// Internal host/device interface between the C ABI (csa_api.cpp) and the
// HIP kernels (csa_kernels.hip).  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

enum Mode { MODE_TOPK = 0, MODE_THRESHOLD = 1, MODE_INTERLEAVED = 2 };

// Queries per workgroup in the generic prefill kernel: 4 waves x 1 query row.
constexpr int PF_ROWS = 4;
constexpr int PF_THREADS = 256;
// Upper bound on the persistent prefill grid (2 workgroups per CU on 256 CUs);
// each workgroup owns one candidate buffer per query row in the workspace.
constexpr int PF_MAX_GRID = 512;
// Keys per LDS stage of the MFMA prefill kernel.
constexpr int PF_KTILE = 64;
// The MFMA prefill kernel (bf16, H = 64, D = 128): 8 waves x 1 query row per
// workgroup in two groups half a step apart, one workgroup per CU, a ring of
// four key-tile stages in LDS.
constexpr int PF2_ROWS = 8;
constexpr int PF2_THREADS = 512;
constexpr int PF2_NSTAGE = 4;
// Query rows per workgroup item of the chosen prefill kernel.
constexpr int prefill_rows_per_block(bool mfma) { return mfma ? PF2_ROWS : PF_ROWS; }

struct PrefillArgs {
  const void* q;
  const void* k;
  const float* w;
  const int32_t* kv_len;
  int B, S_q, T, H, D, m;
  long long q_pos0;
  int causal;
  int kk;               // topk / cap / k_local
  int P;                // partitions (1 unless interleaved)
  int nqb;              // query blocks per (b): ceil(S_q / rows per block)
  int n_items;          // B * nqb * P
  unsigned long long thr_fixed;  // threshold mode: smallest surviving key
  int32_t* out_idx;
  float* out_score;     // may be null
  int32_t* out_count;   // threshold mode
  int out_stride;       // entries per output row (kk, or P*kk when interleaved)
  unsigned long long* cand;      // [grid][rows per block][C] candidate buffers, one per query row
  int C;                // candidate capacity per query row, >= kk + 64
  int need_scores;      // out_score != null
  int bf16;             // element type of q and k: 1 = bf16, 0 = fp32
};

struct DecodeArgs {
  const void* q;
  const void* k;
  const float* w;
  const int32_t* kv_len;
  int B, S_q, T, m;
  long long q_pos0;
  int causal;
  unsigned long long thr_fixed;  // threshold mode: smallest surviving key (0: top-k mode)
  int32_t* out_count;   // threshold mode: survivors per row
  float* scores;        // [B*S_q][dec_row_floats(T)] fp32 workspace
  uint4* bounds;        // [B*S_q][nbw] per-wave selection bounds {order bits, count, max order bits, 0}
  int nbw;              // bounds per row: DEC_THREADS / WAVE per key chunk
  int chunk;            // keys per scan workgroup: DEC_CHUNK or DEC_CHUNK_LONG
  int kk;
  int32_t* out_idx;
  float* out_score;
};

// Up to 8 decode problems of one shape (B, S_q, T) launched together.
constexpr int DEC_MAX_BATCH = 8;
struct DecodeBatch {
  DecodeArgs a[DEC_MAX_BATCH];
  int L;
};

constexpr int DEC_THREADS = 256;
constexpr int DEC_CHUNK = 1024;        // keys per decode-scan workgroup
constexpr int DEC_CHUNK_LONG = 2048;   // ... for long rows with enough workgroups (DecodeArgs::chunk)
constexpr int DEC_RING = 3;            // key-row buffers per wave in the decode scan
constexpr int DEC_PAD = 64;            // floats after each score row (stores of keys past the end)
// Floats per row of the decode score workspace: T rounded up to a multiple of
// 4 (16-byte aligned rows for the select's 16-byte loads) plus the pad.
__host__ __device__ constexpr long long dec_row_floats(int T) { return (((long long)T + 3) & ~3ll) + DEC_PAD; }
constexpr int DEC_SEL_THREADS = 1024;

// Sparse attention over selected keys (H = 64 heads, Dk = Dv = 128, bf16).
constexpr int AT_H = 64, AT_D = 128;
constexpr int AT_CHUNK = 256;          // selected keys per step of a workgroup
constexpr int AT_THREADS = 512;        // 8 waves: 32 keys each for the logits

struct AttnArgs {
  const void* q;        // [rows][AT_H][AT_D] bf16
  const void* k;        // [B][T][AT_D] bf16
  const void* v;        // [B][T][AT_D] bf16
  const int32_t* idx;   // [rows][n_sel]
  int B, S_q, T, n_sel;
  float scale;
  int nsplit;           // workgroups per query row (each takes chunks split, split + nsplit, ...)
  float* opart;         // [rows][nsplit][AT_H][AT_D] unnormalised partial outputs
  float* mpart;         // [rows][nsplit][AT_H] running max (-inf: no valid entry)
  float* lpart;         // [rows][nsplit][AT_H] sum of exp(z - max)
  float* out;           // [rows][AT_H][AT_D]
};

hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

// Per-row union of several index lists (multi-layer selection).
constexpr int UN_MAX_LISTS = 8;
constexpr int UN_MAX_T = 1 << 20;      // keys covered by the LDS bitmap (128 KiB)
constexpr int UN_THREADS = 1024;

// Dense projection y[M][N] = x[M][K] . w[N][K]^T, bf16 operands, fp32
// accumulation, bf16 or fp32 output (the producers of the indexer's inputs).
constexpr int PJ_BK = 64;              // K per pipeline step (K must be a multiple)
struct ProjArgs {
  const void* x;                       // bf16 [M][K]
  const void* w;                       // bf16 [N][K]
  void* y;                             // [M][N], bf16 or fp32
  long long M;
  int N, K;
  int out_f32;
};
hipError_t launch_project(const ProjArgs& a, int variant, hipStream_t st);
long long project_rows_limit();

struct UnionArgs {
  const int32_t* list[UN_MAX_LISTS];   // list i: [rows][width[i]]
  int width[UN_MAX_LISTS];
  int L;
  int T;
  int cap;
  int32_t* out_idx;                    // [rows][cap]
  int32_t* out_count;                  // [rows]
};

hipError_t launch_union(const UnionArgs& a, long long rows, hipStream_t st);

// mfma: the bf16 H=64 D=128 MFMA kernel; otherwise the generic kernel for a.bf16.
hipError_t launch_prefill(const PrefillArgs& a, int mode, bool mfma, int grid, hipStream_t st);
// Resident workgroups per CU of the chosen prefill kernel (>= 1).
int prefill_blocks_per_cu(int mode, bool mfma, bool bf16);
hipError_t launch_decode(const DecodeArgs& a, int nsplit, hipStream_t st);

// Scratch for the no-allocation decode entry point (csa_index_topk_decode_noalloc).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(8) << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
// This device's address of the scratch array (looked up once per device).
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_decode_batch(const DecodeBatch& bt, int nsplit, hipStream_t st);
hipError_t launch_sort_rows(int32_t* idx, float* score, long long rows, int len, hipStream_t st);
hipError_t launch_recall(const int32_t* sel, int n_sel, const int32_t* ref, int n_ref,
                         long long rows, int T, float* out, hipStream_t st);

}  // namespace csa
