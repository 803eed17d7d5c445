/*
 * mla.h -- C ABI of libmla, Multi-head Latent Attention (MLA) for AMD MI355X (gfx950).
 *
 * The operations are those of the notes page "【论文解读】DeepSeek-V3"
 * (wkq9411.github.io), section 一(一) "多头潜在注意力MLA":
 *   c^KV = W^DKV h,  k^C = W^UK c^KV,  v^C = W^UV c^KV              (section 2)
 *   c^Q  = W^DQ h,   q^C = W^UQ c^Q                                  (section 2)
 *   q^R  = RoPE(W^QR c^Q) per head,  k^R = RoPE(W^KR h) shared        (section 3)
 *   o_{t,i} = sum_{j<=t} Softmax_j(q_{t,i} . k_{j,i} / sqrt(d_h + d_h^R)) v_{j,i}
 * with q_{t,i} = [q^C_{t,i}; q^R_{t,i}] and k_{j,i} = [k^C_{j,i}; k^R_j]
 * (the ten-step "完整计算过程" list), and an RMSNorm after each compressed
 * latent (section 二(二)1).  Only c^KV and k^R are cached per token (end of
 * section 一(一)3).  The library computes attention in the absorbed form of
 * the 【思考】 passage on absorption: W_i^UK is folded into the query
 * (q_lat = W_i^UK^T q^C_i, score = q_lat . c_j + q^R_i . k^R_j) and W_i^UV is
 * applied after the weighted sum of latents (o_i = W_i^UV sum_j a_j c_j).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the comment says "host".  The caller
 *    owns and allocates every buffer (cache pool, workspace, outputs); the
 *    library never allocates, frees or synchronises, and keeps no mutable
 *    global state, so calls on different streams may run concurrently as long
 *    as they touch disjoint buffers.  The one exception is
 *    mla_decode_noalloc, whose workspace is a per-GPU array of the library.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  MLA_OK means "enqueued".
 *  - Argument, shape and dtype errors are detected on the host BEFORE any
 *    launch, so a call that returns an error has written nothing.  A launch
 *    failure returns MLA_ERR_HIP.  No C++ exception crosses this interface.
 *  - Weights are row-major [out, in] (y = W x); head i owns rows
 *    [i*w, (i+1)*w) of a per-head projection of width w.
 *  - MLA_BF16: bf16 storage, fp32 accumulation; the hand-written MFMA kernels
 *    serve d_c = 512, d_rope = 64, d_head = 128 and n_heads a multiple of 32
 *    (DeepSeek-V3 shapes).  MLA_F32: fp32 end to end, any small shape
 *    (d_c <= 1024, d_rope <= 128, d_head <= 256, even d_rope).  Other
 *    combinations return MLA_ERR_UNSUPPORTED.
 *  - Pointers must be 16-byte aligned; row widths are in elements.
 *  - Positions are 0-based absolute token positions within a sequence.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 5

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, misalignment */
  MLA_ERR_UNSUPPORTED = 2,  /* shape / dtype combination not implemented   */
  MLA_ERR_OUT_OF_RANGE = 3, /* a host-visible length exceeds the cache      */
  MLA_ERR_WORKSPACE = 4,    /* workspace smaller than *_workspace_size()    */
  MLA_ERR_HIP = 5           /* a HIP launch or runtime call failed          */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Which algebraically equal form mla_prefill computes attention in.
 *  ABSORBED: W_i^UK folded into the query, W_i^UV applied after the weighted
 *            sum of latents (the 【思考】 passage on absorption); scores are
 *            576-wide dot products with the cached rows.
 *  EXPLICIT: k^C = W^UK c and v^C = W^UV c materialised per head for the
 *            sequence's rows (section 2), then causal attention with 192-wide
 *            keys and 128-wide values (the ten-step list as written).  bf16
 *            with d_head = 128 and d_rope = 64 only.
 *  AUTO:     EXPLICIT where supported and it takes fewer FLOPs (long new
 *            chunks), else ABSORBED. */
typedef enum { MLA_PREFILL_AUTO = 0, MLA_PREFILL_ABSORBED = 1, MLA_PREFILL_EXPLICIT = 2 } mla_prefill_form;

/* Layer dimensions (host struct).  Names follow the notes page's symbols. */
typedef struct {
  int32_t n_heads;     /* n_h                                              */
  int32_t d_head;      /* d_h                                              */
  int32_t d_rope;      /* d_h^R, even                                      */
  int32_t d_c;         /* KV latent width d_c                              */
  int32_t d_cq;        /* query latent width d_c'                          */
  int32_t d_model;     /* hidden width d                                   */
  int32_t page_size;   /* tokens per cache page; a multiple of 32          */
  float softmax_scale; /* normally 1/sqrt(d_head + d_rope)                 */
  float rope_base;     /* theta_p = rope_base^(-2p/d_rope)                 */
  float rms_eps;       /* RMSNorm epsilon                                  */
  int32_t dtype;       /* mla_dtype                                        */
  int32_t prefill_form; /* mla_prefill_form (mla_prefill only)             */
  /* YaRN long-context extension (notes page, section 三(二)3: s = 40,
   * alpha = 1, beta = 32, sqrt(t) = 0.1 ln s + 1, original window 4K; the
   * method's meaning from the YaRN paper the page points to).  Off when
   * yarn_s <= 1.  On: every RoPE frequency theta_p (k^R in the cache, q^R in
   * prefill) becomes (1-g) theta_p / s + g theta_p with g = clamp((r - alpha)
   * / (beta - alpha), 0, 1), r = yarn_orig_ctx * theta_p / (2 pi), and every
   * attention logit is multiplied by (0.1 ln s + 1)^2 on top of
   * softmax_scale (prefill and decode).  mla_decode's q_pe must be rotated
   * with the same frequencies by the caller. */
  float yarn_s;
  float yarn_alpha;
  float yarn_beta;
  int32_t yarn_orig_ctx;
  /* FP8 latent cache (0 or 1; MLA_BF16 only).  The notes page, section
   * 二(三) "FP8训练" (fine-grained quantisation), scales activations per
   * 1 x 128 tile; the cache applies that to c^KV: E4M3 codes (OCP "e4m3fn",
   * largest finite 448) with one power-of-two scale 2^e per 128 values, e the
   * smallest integer with max|x| <= 448 * 2^e, codes rounded to nearest, ties
   * to even.  k^R stays bf16.  Attention still computes in bf16 with fp32
   * accumulation on the decoded values.  See mla_kv_cache for the row. */
  int32_t kv_fp8;
} mla_config;

/* Paged latent cache (host struct holding device pointers).
 *  pool        [num_pages, page_size, d_c + d_rope] in cfg->dtype.  Token p
 *              of sequence b lives at pool[block_table[b*max_pages_per_seq
 *              + p/page_size]][p % page_size]; its row is c^KV (RMSNorm'd,
 *              d_c values) followed by k^R (rotated, d_rope values).
 *              With cfg->kv_fp8 a row is 656 bytes: bytes 0..511 the E4M3
 *              codes of c^KV, 512..639 k^R as 64 bf16, 640..655 four fp32
 *              scales 2^e (scale t covers c^KV values 128t .. 128t+127);
 *              value d of c^KV is code(d) * scale(d / 128).
 *              mla_cache_row_bytes() gives the row size for a config.
 *  block_table [n_seqs, max_pages_per_seq] int32 page ids.
 *  err_flags   optional int32 word (may be NULL).  Kernels that meet a page
 *              id outside [0, num_pages), a position beyond the table, or a
 *              length beyond the caller's bound OR a bit into it and skip the
 *              offending row (no out-of-bounds access); see MLA_FLAG_*. */
typedef struct {
  void* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int32_t max_pages_per_seq;
  int32_t* err_flags;
} mla_kv_cache;

#define MLA_FLAG_BAD_PAGE 1 /* block-table entry outside [0, num_pages)        */
#define MLA_FLAG_BAD_POS 2  /* position < 0 or beyond max_pages_per_seq pages  */
#define MLA_FLAG_BAD_LEN 4  /* kv_len < s_q or kv_len > max_kv_len              */
#define MLA_FLAG_BAD_SEQ 8  /* append seq_idx outside [0, n_seqs)              */

/* Layer weights (host struct holding device pointers), all cfg->dtype.
 *  w_dq [d_cq, d_model]          W^DQ     g_q  [d_cq]   RMSNorm gain of c^Q
 *  w_uq [n_heads*d_head, d_cq]   W^UQ     w_qr [n_heads*d_rope, d_cq]  W^QR
 *  w_dkv [d_c, d_model]          W^DKV    g_kv [d_c]    RMSNorm gain of c^KV
 *  w_kr [d_rope, d_model]        W^KR (shared decoupled key)
 *  w_uk, w_uv [n_heads*d_head, d_c]   W^UK, W^UV */
typedef struct {
  const void *w_dq, *g_q, *w_uq, *w_qr, *w_dkv, *g_kv, *w_kr, *w_uk, *w_uv;
} mla_weights;

/* Version of this interface (MLA_ABI_VERSION). */
int32_t mla_abi_version(void);

/* Bytes of one cached row for cfg (host): (d_c + d_rope) elements of
 * cfg->dtype, or 656 with kv_fp8; -1 if cfg fails the checks every entry
 * point makes (see mla_status). */
int64_t mla_cache_row_bytes(const mla_config* cfg);

/* Static, human-readable name of a status code. */
const char* mla_status_string(mla_status status);

/* Cache append (section 一(一)3: only c^KV and k^R are cached; section
 * 二(二)1: RMSNorm after the compressed latent).  For each i < n, writes
 *   [ RMSNorm(ckv_raw[i]; g_kv, rms_eps) ; RoPE(kr_raw[i], pos[i]) ]
 * to the slot of token pos[i] of sequence seq_idx[i].
 *  ckv_raw [n, d_c], kr_raw [n, d_rope] (before rotation), g_kv [d_c]: cfg->dtype.
 *  seq_idx, pos [n] int32 (device).  n_seqs bounds seq_idx (rows of the
 *  block table).  n == 0 is a no-op.  Rows that two i share are written in
 *  unspecified order. */
mla_status mla_cache_append(const mla_config* cfg, const mla_kv_cache* cache,
                            const void* ckv_raw, const void* kr_raw, const void* g_kv,
                            const int32_t* seq_idx, const int32_t* pos, int32_t n,
                            int32_t n_seqs, void* stream);

/* Down-projection of the cached latents, then append (steps (5) and (7) of the
 * complete computation): for token t of sequence b at position start_pos + t,
 *   [c_raw ; k_raw] = [W^DKV ; W^KR] h[b, t]   (one GEMM, fp32 accumulation)
 * followed by the append above.  h [B, L, d_model].  Uses the workspace of
 * mla_project_kv_workspace_size(). */
mla_status mla_project_kv_workspace_size(const mla_config* cfg, int32_t B, int32_t L, size_t* bytes);
mla_status mla_project_kv(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w,
                          const void* h, int32_t B, int32_t L, int32_t start_pos, void* ws,
                          size_t ws_bytes, void* stream);

/* Causal prefill (all ten steps): sequences b < B hold L new tokens at
 * positions [start_pos, start_pos + L).  Appends their rows to the cache
 * (block-table row b), then computes for every new token t and head i
 *   o[b, t, i, :] = W_i^UV sum_{j <= start_pos+t} a_j c_j   (d_head values)
 * over all cached rows of sequence b (rows [0, start_pos) must already be
 * present).  h [B, L, d_model]; out [B, L, n_heads, d_head]; both cfg->dtype.
 * The output stops at o (W^O is not applied).  cfg->prefill_form picks the
 * form of the attention (see mla_prefill_form); both give the same o up to
 * rounding.  MLA_PREFILL_EXPLICIT on a shape it does not serve returns
 * MLA_ERR_UNSUPPORTED.  The explicit form's workspace holds k^C and v^C of
 * rows [0, start_pos + L) of every sequence: B * (start_pos + L) * n_heads *
 * d_head * 4 bytes. */
mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t B, int32_t L, int32_t start_pos,
                                      size_t* bytes);
mla_status mla_prefill(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w,
                       const void* h, int32_t B, int32_t L, int32_t start_pos, void* out, void* ws,
                       size_t ws_bytes, void* stream);

/* Decode step over the paged cache (split-context flash decoding).  Sequence
 * b < B has kv_lens[b] cached rows, the last s_q of which are this step's
 * tokens; query s sits at position kv_lens[b] - s_q + s and attends to rows
 * j <= that position.
 *  kv_lens [B] int32 (device); max_kv_len (host) bounds every kv_lens[b] and
 *          sizes the split plan.
 *  q_nope [B, s_q, n_heads, d_head]   q^C
 *  q_pe   [B, s_q, n_heads, d_rope]   q^R, already rotated
 *  w_uk, w_uv [n_heads*d_head, d_c]
 *  out    [B, s_q, n_heads, d_head]
 * The workspace holds the absorbed queries, the split partials and the merged
 * latent outputs; size it with mla_decode_workspace_size(). */
mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t B, int32_t s_q,
                                     int32_t max_kv_len, size_t* bytes);
mla_status mla_decode(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens,
                      int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope,
                      const void* q_pe, const void* w_uk, const void* w_uv, void* out, void* ws,
                      size_t ws_bytes, void* stream);

/* Output projection (the absorption passage of the notes page: u_t = W^O
 * [o_t,1; ...; o_t,n_h], W_i^O the d_h-column block of head i):
 *   u[t, :] = W^O x[t, :]   for t < T,
 *  x   [T, width]         the heads' outputs concatenated: mla_prefill's or
 *                         mla_decode's out viewed as [T, n_heads * d_head]
 *  w_o [d_model, width]   W^O (width = n_heads * d_head), or the fold
 *                         W^O' = [W_1^O W_1^UV, ...] of the same passage
 *                         (width = n_heads * d_c, applied to the latent
 *                         sums o^lat instead of o)
 *  u   [T, d_model]
 * All cfg->dtype; width a multiple of 64, d_model a multiple of 8.  Small T
 * splits the reduction over width (fp32 partials in the workspace, summed
 * in a second pass); size the workspace with
 * mla_output_projection_workspace_size(). */
mla_status mla_output_projection_workspace_size(const mla_config* cfg, int32_t T, int32_t width, size_t* bytes);
mla_status mla_output_projection(const mla_config* cfg, const void* x, int32_t width, const void* w_o, void* u,
                                 int32_t T, void* ws, size_t ws_bytes, void* stream);

/* Measurement variants: identical to mla_decode / mla_prefill, and in
 * addition record attn_start and attn_stop (hipEvent_t, either may be NULL) on
 * `stream` immediately before and after the latent-attention kernel, so a
 * caller can time that kernel alone with hipEventElapsedTime. */
mla_status mla_decode_profiled(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens,
                               int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, void* out, void* ws, size_t ws_bytes,
                               void* stream, void* attn_start, void* attn_stop);
mla_status mla_prefill_profiled(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w,
                                const void* h, int32_t B, int32_t L, int32_t start_pos, void* out, void* ws,
                                size_t ws_bytes, void* stream, void* attn_start, void* attn_stop);

/* Decode without allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, checks and result as mla_decode, without the
 * workspace: the library keeps one scratch array of
 * MLA_DECODE_NOALLOC_SCRATCH_BYTES in the memory of each GPU it is loaded on
 * (held until the process ends) and carves the decode workspace out of it.
 * When the usual workspace for these sizes does not fit, fewer split slots
 * are used (the plan then cuts ragged batches into fewer, longer chunks; the
 * result is the same up to rounding); when even that does not fit (with
 * the V3 shapes and 64-token pages: more than 336 query rows B * s_q, fewer
 * for contexts past 98,240 tokens, e.g. 252 at 131,073) the call returns
 * MLA_ERR_WORKSPACE before any launch.  Nothing in the array needs to start at zero: every call
 * writes its plan, queries and partials before reading them.
 *  - The array is shared by every call on a GPU and keeps the last call's
 *    contents: calls that overlap on one GPU (different streams without
 *    ordering, or threads) race and corrupt each other's results.  Serialise
 *    them (one stream, or events).
 *  - `stream` must belong to the current device (MLA_ERR_INVALID_ARG if not).
 *  - No hipMalloc, hipFree or other allocating call is made; the first call on
 *    a device looks up the array's device address (hipGetSymbolAddress). */
#define MLA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
mla_status mla_decode_noalloc(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens,
                              int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope, const void* q_pe,
                              const void* w_uk, const void* w_uv, void* out, void* stream);

/* Measurement helper (not part of the attention arithmetic): read `bytes`
 * bytes of device memory at src once, as a plain streaming kernel, so a
 * caller can time the HBM read ceiling the decode kernel is compared with.
 * bytes > 0 and src 16-byte aligned, else MLA_ERR_INVALID_ARG.  `sink` (may
 * be NULL, else one writable uint32) is written only in the practically
 * impossible case that the XOR of all words read equals 0x9E3779B9. */
mla_status mla_stream_read(const void* src, int64_t bytes, void* sink, void* stream);

/* Measurement helper (not part of the attention arithmetic): the sustained
 * bf16 matrix-core rate on this device.  One workgroup of four waves per CU;
 * each wave loads its operand fragments once from `operands` (bf16 values,
 * e.g. random: the rate depends on the operands' switching activity), then
 * issues `iters` rounds of independent MFMAs into 256 fp32 accumulators:
 * shape 16 = v_mfma_f32_16x16x32_bf16 (64 per round), shape 32 =
 * v_mfma_f32_32x32x16_bf16 (32 per round); 2^20 FLOP per wave per round for
 * both.  operands 16-byte aligned with bytes >= 262144 (fragments past the
 * end wrap around), iters > 0, shape 16 or 32, else MLA_ERR_INVALID_ARG.
 * `sink` (may be NULL, else one writable float) is written only in the
 * practically impossible case that the accumulators' sum is exactly
 * 1234567.0.  `clocks` (may be NULL, else two 8-byte-aligned uint64 on the
 * device, which the caller zeroes) receives, summed over the workgroups,
 * the core-clock cycles (s_memtime) and the 100 MHz ticks (s_memrealtime)
 * each spent in its MFMA rounds: 0.1 * clocks[0] / clocks[1] is the average
 * core clock in GHz under the stream (the matrix cores run at the part's
 * power limit, below the 2.4 GHz peak clock).  A misaligned clocks pointer
 * gives MLA_ERR_INVALID_ARG. */
mla_status mla_mfma_rate(const void* operands, int64_t bytes, int32_t iters, int32_t shape, void* sink,
                         void* clocks, void* stream);

/* Upper bound on the attention work items (split partial slots) mla_decode
 * plans for these sizes; the device plan cuts each query row's visible keys
 * into chunks from the actual kv_lens.  Host helper for tests and sizing;
 * returns 0 for invalid arguments. */
int32_t mla_decode_num_splits(const mla_config* cfg, int32_t B, int32_t s_q, int32_t max_kv_len);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
