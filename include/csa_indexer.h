/*
 * csa_indexer.h -- C ABI of the MI355X (gfx950) CSA lightning-indexer top-k library.
 *
 * The operation.  DeepSeek-V3.2/V4 Compressed Sparse Attention (CSA) scores
 * every compressed key with a "lightning indexer" and keeps the top-k keys of
 * each query; the attention step that follows touches only the selected keys
 * ("StreamIndex: Memory-Bounded Compressed Sparse Attention via Streaming
 * Top-k", abstract).  The indexer score is a per-head dot product of the query
 * with the compressed key, passed through ReLU and fused across heads with
 * per-head weights ("FlashMemory-DeepSeek-V4" machine review, axiom ledger,
 * Eq. 4 as cited there; its "What carries the argument" section names ReLU as
 * the native Lightning Indexer activation):
 *
 *     I[b,t,s] = sum_{j<H} w[b,t,j] * max( sum_{d<D} q[b,t,j,d] * k[b,s,d], 0 )
 *
 * Keys are compressed by ratio m (V4-Flash: m = 4, StreamIndex abstract); the
 * query at absolute position t = q_pos0 + i sees keys s <= floor(t/m) (and
 * s < T, s < kv_len[b]).  Selection is an exact top-k in the total order
 * (score descending, key index ascending); -0.0 scores equal +0.0.  The
 * library streams over keys and never forms the [B,S,H,T] score tensor that
 * StreamIndex's abstract identifies as the memory problem (256 GB at
 * S = 65,536, H = 64, m = 4).
 *
 * Conventions for every entry point:
 *  - Pointers to tensors are DEVICE pointers unless marked (host).  Tensors
 *    are packed row-major with the last dimension contiguous.
 *  - The caller owns every buffer.  The library never allocates device memory
 *    and never synchronises; work is enqueued on `hip_stream` (a hipStream_t;
 *    NULL = the null stream) and the call returns at once.
 *  - Argument validation is synchronous: on any error nothing is enqueued and
 *    a non-zero csa_status is returned; csa_last_error() gives a message
 *    (thread-local).  No C++ exception crosses this interface.
 *  - Outputs are deterministic (bitwise identical for identical inputs and
 *    launch configuration).  out_idx rows are SETS: entry order is unspecified
 *    unless CSA_SORTED is given, which orders them by (score desc, index asc).
 *    Rows with fewer than topk visible keys hold all visible keys first, then -1;
 *    out_score (optional, may be NULL) holds the fp32 score of each entry and
 *    -INFINITY for padding.
 *  - Workspace: `ws` must hold at least csa_workspace_size(...) bytes for the
 *    same problem, flags and device and be 16-byte aligned (CSA_ERR_INVALID
 *    otherwise); it needs no initialisation and its contents are undefined
 *    after the call.  ws may be NULL when that size is 0.
 *  - Calls that share a workspace must not overlap (same stream = safe).
 *  - Library state.  Besides the thread-local error string the library keeps
 *    (a) a per-device count of resident prefill workgroups per compute unit,
 *    asked once per device and kernel variant from the HIP occupancy API and
 *    only read afterwards (a mutex guards the first fill), (b) the test
 *    options of csa_set_test_option, and (c) per GPU, the scratch array of
 *    csa_index_topk_decode_noalloc and its address, looked up once.  Entry points are otherwise stateless
 *    and may be called from several threads on different streams.
 */
#ifndef CSA_INDEXER_H
#define CSA_INDEXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID = 1,     /* bad argument: null pointer, size <= 0, bad struct_size, ... */
  CSA_ERR_UNSUPPORTED = 2, /* valid but not compiled: D, H, topk beyond limits, T >= 2^31 */
  CSA_ERR_WORKSPACE = 3,   /* ws_bytes smaller than csa_workspace_size() */
  CSA_ERR_DEVICE = 4       /* a HIP call or kernel launch failed */
} csa_status;

typedef enum { CSA_BF16 = 0, CSA_F32 = 1 } csa_dtype; /* dtype of q and k; w is always fp32 */

enum {
  CSA_SORTED = 1u,    /* order each output row by (score desc, index asc) */
  CSA_NONCAUSAL = 2u  /* every key s < T (and < kv_len[b]) is visible */
};

/* Operation codes for csa_workspace_size. */
enum {
  CSA_OP_PREFILL = 0,
  CSA_OP_DECODE = 1,
  CSA_OP_THRESHOLD = 2,
  CSA_OP_INTERLEAVED = 3,
  CSA_OP_RECALL = 4
};

/* Limits of this library version. */
#define CSA_MAX_TOPK 4096   /* topk, cap and k_local */
#define CSA_MAX_HEADS 128
#define CSA_MAX_DECODE_SQ 16

/* Problem description (host struct, passed by pointer).  Shapes:
 *   q [B, S_q, H, D]  (dtype)      one query row per token, H indexer heads
 *   k [B, T, D]       (dtype)      compressed keys
 *   w [B, S_q, H]     fp32         per-query head weights
 *   kv_len [B] int32 or NULL       extra per-sequence cap on visible keys
 * D must be one of 32, 64, 128, 256; 1 <= H <= CSA_MAX_HEADS; T < 2^31.   */
typedef struct {
  uint32_t struct_size; /* must equal sizeof(csa_problem) */
  int32_t dtype;        /* csa_dtype */
  int32_t B, S_q, T, H, D;
  int32_t m;            /* compression ratio, >= 1 */
  int64_t q_pos0;       /* absolute position of query row 0, >= 0 */
  const void* q;
  const void* k;
  const float* w;
  const int32_t* kv_len;
} csa_problem;

/* Bytes of workspace the given operation needs on the current device.
 * op: CSA_OP_*.  k_or_cap: topk (PREFILL, DECODE), cap (THRESHOLD) or k_local
 * (INTERLEAVED); P: partitions (INTERLEAVED, else ignored).  For CSA_OP_RECALL
 * pass prob = NULL; the size is 0.  bytes (host) receives the size. */
csa_status csa_workspace_size(int op, const csa_problem* prob, int32_t k_or_cap, int32_t P,
                              uint32_t flags, size_t* bytes);

/* Top-k key indices per query row (StreamIndex abstract: every query keeps
 * its own top-k keys), streaming over key tiles with a running per-query
 * threshold; any S_q.  out_idx [B, S_q, topk] int32; out_score [B, S_q, topk]
 * fp32 or NULL.  1 <= topk <= CSA_MAX_TOPK. */
csa_status csa_index_topk_prefill(const csa_problem* prob, int32_t topk, uint32_t flags,
                                  int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                  void* hip_stream);

/* Same contract and same result sets as csa_index_topk_prefill, for a few
 * query rows per sequence against a long key range (decode: S_q <=
 * CSA_MAX_DECODE_SQ).  The key scan is split across many workgroups and is
 * bound by HBM bandwidth; the multi-layer-indexer blog post (rit.work) reports
 * the indexer scan at about two thirds of a layer's attention-part time in
 * 128K-context decode. */
csa_status csa_index_topk_decode(const csa_problem* prob, int32_t topk, uint32_t flags,
                                 int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                 void* hip_stream);

/* csa_index_topk_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, limits and
 * results as csa_index_topk_decode; the decode workspace comes from a fixed
 * scratch array of CSA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on until the process ends, so the call allocates nothing.
 * Supported: the decode fast path (bf16 q and k, H = 64, D = 128, S_q <=
 * CSA_MAX_DECODE_SQ) with a workspace need of at most the scratch size, i.e.
 * about B*S_q*(T+67)*4 bytes of scores plus 64 bytes per 1024 keys per row
 * (B*S_q = 32 rows at T = 32768 take 4.2 MB); larger problems and other
 * shapes return CSA_ERR_UNSUPPORTED with nothing enqueued.  The scratch needs
 * no initialisation.  Every call on one GPU uses that GPU's one array: calls
 * that overlap on one GPU (different streams, or other threads) race and
 * give undefined results; calls in one stream are ordered and safe. */
#define CSA_NOALLOC_SCRATCH_BYTES (8u << 20)
csa_status csa_index_topk_decode_noalloc(const csa_problem* prob, int32_t topk, uint32_t flags,
                                         int32_t* out_idx, float* out_score, void* hip_stream);

/* Sigmoid-threshold selection (FlashMemory-DeepSeek-V4 review, "What carries
 * the argument": in place of a top-k of fixed size, its Memory Indexer keeps
 * every key whose score, after a sigmoid, is above 0.5).  Read as
 * sigmoid(I + logit_bias) > prob_threshold, i.e. I > logit(tau) - bias
 * (strict), decided on the fp32 score.  0 < prob_threshold < 1.
 * out_count [B, S_q] int32: the true number of survivors (may exceed cap).
 * out_idx [B, S_q, cap]: the min(cap, count) best survivors (score desc,
 * index asc define "best"), then -1.  out_score optional. */
csa_status csa_index_threshold_select(const csa_problem* prob, float prob_threshold,
                                      float logit_bias, int32_t cap, uint32_t flags,
                                      int32_t* out_idx, int32_t* out_count, float* out_score,
                                      void* ws, size_t ws_bytes, void* hip_stream);

/* Interleaved relaxed selection on one GPU (Machine Press, "Million-Token
 * Memory Without the Global Bottleneck": tokens laid out interleaved across
 * devices, each device selects locally, the union is meant to cover the
 * global top tokens).  Partition p < P holds keys s with s mod P == p and
 * keeps its own top-k_local.  out_idx [B, S_q, P*k_local]: partition p's set
 * at offset p*k_local, padded with -1.  out_score optional, same layout. */
csa_status csa_index_topk_interleaved(const csa_problem* prob, int32_t P, int32_t k_local,
                                      uint32_t flags, int32_t* out_idx, float* out_score,
                                      void* ws, size_t ws_bytes, void* hip_stream);

/* Union recall of a selection against a reference selection, per row:
 * |set(sel) ∩ set(ref)| / |set(ref)|, entries < 0 ignored; 1.0 when ref has
 * no valid entry.  sel [rows, n_sel], ref [rows, n_ref] int32;
 * out_recall [rows] fp32.  1 <= n_ref <= 8192, n_sel >= 1, T bounds valid
 * indices (entries >= T are ignored).  ws unused (may be NULL). */
csa_status csa_set_recall(const int32_t* sel, int32_t n_sel, const int32_t* ref, int32_t n_ref,
                          int64_t rows, int32_t T, float* out_recall, void* ws, size_t ws_bytes,
                          void* hip_stream);

/* Sparse attention over the selected keys: the CSA step that consumes the
 * indexer's out_idx (StreamIndex abstract: the attention step of CSA reads
 * only the keys the indexer picks; the Multi-layer Indexer blog post: each
 * DeepSeek Sparse Attention layer attends to the 2048 entries its indexer
 * picks).  The pages give no formula for this step; it is read as scaled
 * softmax attention in which every query head attends to the same selected
 * compressed key and value rows:
 *
 *   o[b,t,h,:] = sum_e p_e v[b, idx[b,t,e], :],
 *   p = softmax_e( scale * q[b,t,h,:] . k[b, idx[b,t,e], :] )
 *
 * over the entries e of idx[b,t,0:n_sel] with 0 <= idx < T (others skipped;
 * an index listed twice counts twice); a row with no valid entry gives 0.
 * q [B,S_q,H,Dk], k [B,T,Dk], v [B,T,Dv] bf16; idx [B,S_q,n_sel] int32 (for
 * example out_idx of a top-k call); out [B,S_q,H,Dv] fp32.  Supported:
 * H = 64, Dk = Dv = 128 (CSA_ERR_UNSUPPORTED otherwise); n_sel >= 1; scale
 * finite.  Computed in fp32 from bf16 inputs with the softmax weights rounded
 * to bf16 for the weighted sum of value rows. */
typedef struct {
  uint32_t struct_size; /* must equal sizeof(csa_attn_problem) */
  int32_t B, S_q, T, H, Dk, Dv;
  const void* q;
  const void* k;
  const void* v;
} csa_attn_problem;

/* Workspace bytes of csa_sparse_attention for this problem and n_sel. */
csa_status csa_attention_workspace_size(const csa_attn_problem* prob, int32_t n_sel, size_t* bytes);

csa_status csa_sparse_attention(const csa_attn_problem* prob, const int32_t* idx, int32_t n_sel, float scale,
                                float* out, void* ws, size_t ws_bytes, void* hip_stream);

/* The threshold selection of several problems of one shape at once (one
 * problem per indexer layer, as in multi-layer selection below): problem i is
 * probs[i], with its results in out_idx[i] [B, S_q, cap] and out_count[i]
 * [B, S_q] (optional out_score[i], or out_score NULL).  probs, out_idx,
 * out_count and out_score are HOST arrays of L entries; 1 <= L <=
 * CSA_MAX_UNION_LISTS.  Same results as L calls of csa_index_threshold_select;
 * the problems run in one launch of each decode kernel, so this form requires
 * what that path requires of every problem (bf16, H=64, D=128, S_q <=
 * CSA_MAX_DECODE_SQ) and equal B, S_q and T (CSA_ERR_UNSUPPORTED otherwise).
 * ws: L times csa_workspace_size(CSA_OP_THRESHOLD, probs[0], cap, ...) bytes. */
csa_status csa_index_threshold_select_layers(const csa_problem* const* probs, int32_t L, float prob_threshold,
                                             float logit_bias, int32_t cap, uint32_t flags, int32_t* const* out_idx,
                                             int32_t* const* out_count, float* const* out_score, void* ws,
                                             size_t ws_bytes, void* hip_stream);

/* Dense projection y[M][N] = x[M][K] . w[N][K]^T with bf16 operands and
 * fp32 accumulation: the producers of the indexer's inputs.  The FlashMemory
 * review gives the Memory Indexer's query encoder a low-rank projection of
 * dimension r = 2048; StreamIndex (abstract) scores keys compressed by a ratio
 * m.  With x and w as below this computes, in the layouts the indexer entry
 * points read (row-major, no conversion pass):
 *   query        x = latents c [B*S][r],       w = W_q [H*D][r]   -> q [B,S,H,D] (bf16)
 *   head weights x = hidden states [B*S][d],   w = W_w [H][d]     -> w [B,S,H]   (fp32)
 *   compressed   x = token vectors [B*S/m][m*d_z] (the m tokens of a group
 *   keys           side by side), w = W_k [D][m*d_z]              -> k [B,T,D]   (bf16)
 * x: DEVICE bf16 [M][K], w: DEVICE bf16 [N][K], both row-major and 16-byte
 * aligned; y: DEVICE [M][N] row-major, bf16 (round to nearest even) when
 * out_dtype = CSA_BF16, fp32 when CSA_F32.  Caller owns all buffers; nothing
 * is allocated; asynchronous on hip_stream.
 * Errors: CSA_ERR_INVALID (NULL pointers with M > 0, M < 0, N or K < 1, bad
 * out_dtype, misalignment); CSA_ERR_UNSUPPORTED (K not a multiple of 64,
 * N > CSA_MAX_PROJECT_N, M above 2^31 - 256).  M = 0 is a no-op. */
#define CSA_MAX_PROJECT_N (1 << 20)
csa_status csa_project(const void* x, const void* w, int64_t M, int32_t N, int32_t K, int32_t out_dtype, void* y,
                       void* hip_stream);

/* Union of several selections per row (multi-layer selection: the
 * FlashMemory-DeepSeek-V4 review, "What carries the argument", places its
 * Memory Indexer on three layers and combines their keep decisions with a
 * logical OR while decoding).  For each of `rows` rows: the set of distinct
 * values v with 0 <= v < T found in row r of any of the L lists (list i is a
 * device array [rows, widths[i]] int32; other entries are ignored), written
 * to out_idx [rows, cap] in ascending order, then -1; out_count [rows]
 * (optional, may be NULL) receives the true size of the union, which may
 * exceed cap (then the cap smallest indices are written).  lists and widths
 * are HOST arrays of L entries; 1 <= L <= CSA_MAX_UNION_LISTS; 1 <= T <=
 * CSA_MAX_UNION_T (CSA_ERR_UNSUPPORTED above); cap >= 1.  No workspace. */
#define CSA_MAX_UNION_LISTS 8
#define CSA_MAX_UNION_T (1 << 20)
csa_status csa_union_rows(const int32_t* const* lists, const int32_t* widths, int32_t L, int64_t rows,
                          int32_t T, int32_t cap, int32_t* out_idx, int32_t* out_count, void* hip_stream);

/* Test options: process-wide switches that let tests drive every code path
 * from one process.  They change which kernel variant runs or how often the
 * prefill candidate lists are compacted, never the results; all are 0 (off,
 * automatic) at load.  Not meant for production use; set them only while no
 * other thread is inside a library call.
 *   CSA_OPT_FORCE_GENERIC  1: every prefill-family call uses the generic
 *                          kernel (one score per lane, fp32 FMAs in index
 *                          order), also for bf16 H = 64, D = 128.
 *   CSA_OPT_CAND_CAP       > 0: candidate keys held per query row between
 *                          compactions of the prefill kernels (raised to the
 *                          minimum 2*k + 64 when smaller); 0: 12*k + 64.
 *   CSA_OPT_DECODE_CHUNK   1024 or 2048: keys per decode-scan workgroup;
 *                          0: chosen from the shape.
 * Errors: CSA_ERR_INVALID for an unknown option or a value outside its range
 * (the option keeps its value). */
enum { CSA_OPT_FORCE_GENERIC = 1, CSA_OPT_CAND_CAP = 2, CSA_OPT_DECODE_CHUNK = 3 };
csa_status csa_set_test_option(int32_t option, int64_t value);

const char* csa_status_str(csa_status s); /* static string, never NULL */
const char* csa_last_error(void);         /* thread-local detail of this thread's last error */
int csa_version(void);                    /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* CSA_INDEXER_H */
