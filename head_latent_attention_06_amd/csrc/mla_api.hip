// C ABI of libmla: argument validation (before any launch), workspace
// carving and the launch sequence of each entry point.  Declarations and the
// contract are in include/mla.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "mla.h"
#include "mla_kernels.h"

using namespace mla;

namespace {

constexpr int ATTN_SPLIT_PAGES = 1536;  // page ids one attention workgroup stages in LDS
constexpr int ATTN_SPLIT_PAGES_FP8 = 512;  // the same with an FP8 cache (its staging takes the LDS)
constexpr int DECODE_TARGET_ITEMS = 256;  // about one workgroup per CU for even batches
constexpr int RAGGED_FACTOR = 4;          // the plan uses 4x as many chunks for ragged ones
constexpr int MIN_CHUNK = 256;
constexpr int MERGE_WUV_MAX_ROWS = 256;   // above this the merge and a W^UV GEMM run separately

struct Carve {
  unsigned char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((unsigned char*)b) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

RopeParams rope_params(const mla_config* c) {
  RopeParams r{};
  r.base = c->rope_base;
  r.yarn_s = c->yarn_s > 1.f ? c->yarn_s : 0.f;
  r.yarn_alpha = c->yarn_alpha;
  r.yarn_beta = c->yarn_beta;
  r.yarn_orig = c->yarn_orig_ctx;
  return r;
}

// softmax_scale times the YaRN logit factor (0.1 ln s + 1)^2 when YaRN is on
float logit_scale(const mla_config* c) {
  if (!(c->yarn_s > 1.f)) return c->softmax_scale;
  const double f = 0.1 * log((double)c->yarn_s) + 1.0;
  return (float)((double)c->softmax_scale * f * f);
}

mla_status check_cfg(const mla_config* c, bool* bf16) {
  if (!c) return MLA_ERR_INVALID_ARG;
  if (c->n_heads <= 0 || c->d_head <= 0 || c->d_rope <= 0 || c->d_c <= 0 || c->d_cq <= 0 || c->d_model <= 0 ||
      c->page_size <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!(c->softmax_scale > 0.f) || !(c->rope_base > 0.f) || !(c->rms_eps >= 0.f)) return MLA_ERR_INVALID_ARG;
  if (c->prefill_form < MLA_PREFILL_AUTO || c->prefill_form > MLA_PREFILL_EXPLICIT) return MLA_ERR_INVALID_ARG;
  if (c->yarn_s > 1.f && !(c->yarn_beta > c->yarn_alpha && c->yarn_orig_ctx > 0)) return MLA_ERR_INVALID_ARG;
  if (c->kv_fp8 != 0 && c->kv_fp8 != 1) return MLA_ERR_INVALID_ARG;
  if (c->kv_fp8 && c->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (c->page_size % 32 != 0 || (c->d_rope & 1)) return MLA_ERR_UNSUPPORTED;
  if (c->dtype == MLA_BF16) {
    *bf16 = true;
    if (c->d_c != 512 || c->d_rope != 64 || c->n_heads % 32 != 0 || c->d_head % 64 != 0 || c->d_head > 512 ||
        c->d_model % 64 != 0 || c->d_cq % 64 != 0)
      return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
  }
  if (c->dtype == MLA_F32) {
    *bf16 = false;
    if (c->d_c > 1024 || c->d_rope > 128 || c->d_head > 256) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
  }
  return MLA_ERR_UNSUPPORTED;
}

mla_status check_cache(const mla_config* c, const mla_kv_cache* k) {
  if (!k || !k->pool || !k->block_table || k->num_pages <= 0 || k->max_pages_per_seq <= 0)
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(k->pool)) return MLA_ERR_INVALID_ARG;
  (void)c;
  return MLA_OK;
}

int32_t max_chunk_keys(const mla_config* c) {
  const int64_t m = (int64_t)((c->kv_fp8 ? ATTN_SPLIT_PAGES_FP8 : ATTN_SPLIT_PAGES) - 1) * c->page_size;
  return (int32_t)(m > (1 << 30) ? (1 << 30) : m);
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound on plan items for n_rows rows of at most max_kv visible keys.
// Chunks capped at max_chunk_keys: at most n_rows * ceil(max_kv / cap).  Else
// chunks of at least max(MIN_CHUNK, T / tgt) keys for T visible keys in all
// and tgt <= target * RAGGED_FACTOR: a row of v keys takes at most
// v / chunk + 1 of them, so n_rows + min(tgt, T / MIN_CHUNK) in all.
int64_t max_plan_items(const mla_config* c, int64_t n_rows, int32_t max_kv, int32_t target) {
  const int64_t by_cap = n_rows * ceil_div(max_kv, max_chunk_keys(c));
  int64_t spread = (int64_t)target * RAGGED_FACTOR;
  if (ceil_div(n_rows * (int64_t)max_kv, MIN_CHUNK) < spread) spread = ceil_div(n_rows * (int64_t)max_kv, MIN_CHUNK);
  const int64_t by_target = target > 0 ? n_rows + spread : 0;
  const int64_t m = by_target > by_cap ? by_target : by_cap;
  // the attention grid spreads the items over the 8 XCDs in equal runs, which
  // can leave up to 7 empty slots: round up to whole rounds of 8
  return m > 0 ? (m + 7 + 7) / 8 * 8 : 0;
}

// ----- workspace layouts --------------------------------------------------
struct DecodeWs {
  void *q_lat, *o_lat, *part_o;
  int32_t* plan;
  float* part_ml;
  int64_t max_items;
};

// items > 0: that many split slots instead of the bound for these sizes
DecodeWs decode_layout(const mla_config* c, bool bf16, int32_t B, int32_t s_q, int32_t max_kv, void* ws,
                       size_t* total, int64_t items = 0) {
  Carve cv(ws);
  DecodeWs d{};
  const int64_t rows = (int64_t)B * s_q, H = c->n_heads, row = c->d_c + c->d_rope;
  const size_t e = bf16 ? 2 : 4;
  d.q_lat = cv.take(rows * H * c->d_c * e);
  d.o_lat = cv.take(rows * H * c->d_c * e);
  if (bf16) {
    d.max_items = items > 0 ? items : max_plan_items(c, rows, max_kv, DECODE_TARGET_ITEMS);
    d.plan = (int32_t*)cv.take(plan_ints(rows, d.max_items) * 4);
    d.part_o = cv.take(d.max_items * H * c->d_c * 2);
    d.part_ml = (float*)cv.take(d.max_items * H * 2 * 4);
  }
  (void)row;
  *total = cv.off;
  return d;
}

// The explicit prefill form: bf16 with the head widths its kernel is built for.
bool explicit_supported(const mla_config* c, bool bf16) { return bf16 && c->d_head == 128 && c->d_rope == 64; }

// Form of the prefill attention.  FLOPs per head beyond the shared projections
// (S cached rows, L new ones, pairs = L S + L (L + 1) / 2):
//   explicit  2 * 2 * d_c * d_h * (S + L)  +  2 (d_h + d_h^R + d_h) pairs
//   absorbed  2 * 2 * d_c * d_h * L        +  2 (d_c + d_h^R + d_c) pairs
// so with V3 widths the explicit form is cheaper once 768 L (2 S + L) >= 262144 S.
mla_status prefill_form(const mla_config* c, bool bf16, int32_t L, int32_t start_pos, bool* use_explicit) {
  const bool ok = explicit_supported(c, bf16);
  if (c->prefill_form == MLA_PREFILL_EXPLICIT) {
    if (!ok) return MLA_ERR_UNSUPPORTED;
    *use_explicit = true;
  } else if (c->prefill_form == MLA_PREFILL_ABSORBED) {
    *use_explicit = false;
  } else {
    // explicit - absorbed = 4 d_c d_h S - 4 (d_c - d_h) pairs
    const int64_t S = start_pos;
    const int64_t pairs = (int64_t)L * S + (int64_t)L * (L + 1) / 2;
    *use_explicit = ok && (int64_t)c->d_c * c->d_head * S <= (int64_t)(c->d_c - c->d_head) * pairs;
  }
  return MLA_OK;
}

// [W^DKV ; W^KR] h has few output columns (d_c + d_rope): with fewer
// 256 x 192 tiles than CUs it runs in the stream-K form: kv_sk_groups()
// groups of one workgroup per column tile (at most SK_MAX_WGS workgroups in
// all, a multiple of 8 groups so each XCD holds whole groups, each group
// with at least SK_MIN_SLICES k slices) share its (row tile, k slice) units
// equally and write partial sums that the append adds.  kv_parts() is the
// number of partial buffers (1: one plain product).
constexpr int SK_MAX_WGS = 256, SK_MIN_SLICES = 48;
int kv_sk_groups(const mla_config* c, bool bf16, int64_t T) {
  const int64_t tiles_m = ceil_div(T, GEMM_SK_BM), tiles_n = ceil_div(c->d_c + c->d_rope, GEMM_SK_BN);
  if (!bf16 || c->d_model % GEMM_SK_BK != 0 || T < GEMM_SK_BM || tiles_m * tiles_n >= SK_MAX_WGS) return 0;
  int64_t g = std::min<int64_t>(SK_MAX_WGS / tiles_n, tiles_m * (c->d_model / GEMM_SK_BK) / SK_MIN_SLICES);
  if (g >= 8) g = g / 8 * 8;
  return g > tiles_m ? (int)g : 0;
}
int kv_parts(const mla_config* c, bool bf16, int64_t T) {
  const int G = kv_sk_groups(c, bf16, T);
  if (!G) return 1;
  const int64_t tiles_m = ceil_div(T, GEMM_SK_BM), nk = c->d_model / GEMM_SK_BK;
  int p = 1;
  for (int64_t t = 0; t < tiles_m; ++t) p = std::max(p, gemm_sk_parts(t, nk, tiles_m * nk, G));
  return p;
}

struct PrefillWs {
  float *kv_raw, *cq_raw, *qr_raw, *rope_cs, *part_ml;
  void *cq, *qc, *q_abs, *o_lat, *part_o;
  void *qr, *kvg, *kc, *vc;  // explicit form
  int32_t* plan;
  int64_t max_items;
  bool split, use_explicit;
};

PrefillWs prefill_layout(const mla_config* c, bool bf16, bool use_explicit, int32_t B, int32_t L, int32_t start_pos,
                         void* ws, size_t* total) {
  Carve cv(ws);
  PrefillWs p{};
  p.use_explicit = use_explicit;
  const int64_t T = (int64_t)B * L, H = c->n_heads, row = c->d_c + c->d_rope;
  const size_t e = bf16 ? 2 : 4;
  p.rope_cs = (float*)cv.take((int64_t)L * c->d_rope * 4);
  p.kv_raw = (float*)cv.take(kv_parts(c, bf16, T) * T * row * 4);
  p.cq_raw = (float*)cv.take(T * c->d_cq * 4);
  p.cq = cv.take(T * c->d_cq * e);
  p.qc = cv.take(T * H * c->d_head * e);
  p.qr_raw = (float*)cv.take(T * H * c->d_rope * 4);
  if (use_explicit) {
    const int64_t nk = (int64_t)B * (start_pos + L);
    p.qr = cv.take(T * H * c->d_rope * e);
    p.kvg = cv.take(nk * row * e);
    p.kc = cv.take(nk * H * c->d_head * e);
    p.vc = cv.take(nk * H * c->d_head * e);
    *total = cv.off;
    return p;
  }
  p.q_abs = cv.take(T * H * row * e);
  p.o_lat = cv.take(T * H * c->d_c * e);
  if (bf16) {
    const int32_t kv_end = start_pos + L;
    p.split = kv_end > max_chunk_keys(c);
    p.max_items = max_plan_items(c, T, kv_end, 0);
    p.plan = (int32_t*)cv.take(plan_ints(T, p.max_items) * 4);
    if (p.split) {
      p.part_o = cv.take(p.max_items * H * c->d_c * 2);
      p.part_ml = (float*)cv.take(p.max_items * H * 2 * 4);
    }
  }
  *total = cv.off;
  return p;
}

size_t project_kv_layout(const mla_config* c, bool bf16, int32_t B, int32_t L, void* ws, float** rope_cs,
                         float** kv_raw) {
  Carve cv(ws);
  const int64_t T = (int64_t)B * L;
  *rope_cs = (float*)cv.take((int64_t)L * c->d_rope * 4);
  *kv_raw = (float*)cv.take(kv_parts(c, bf16, T) * T * (c->d_c + c->d_rope) * 4);
  return cv.off;
}

#define MLA_HIP(x)                          \
  do {                                      \
    if ((x) != hipSuccess) return MLA_ERR_HIP; \
  } while (0)

mla_status launch_gemm(bool bf16, const GemmArgs& g, hipStream_t st) {
  MLA_HIP(bf16 ? launch_gemm_bf16(g, st) : launch_gemm_f32(g, st));
  return MLA_OK;
}

GemmArgs gemm(const void* A, int64_t lda, int64_t sA, const void* B, int64_t ldb, int64_t sB, void* C, int64_t ldc,
              int64_t sC, int M, int N, int K, int batch, bool b_kn, bool out_bf16) {
  GemmArgs g{};
  g.A = A; g.lda = lda; g.strideA = sA;
  g.B = B; g.ldb = ldb; g.strideB = sB;
  g.B2 = nullptr; g.n_split = 0;
  g.C = C; g.ldc = ldc; g.strideC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch;
  g.b_kn = b_kn ? 1 : 0;
  g.out_bf16 = out_bf16 ? 1 : 0;
  return g;
}

// [c_raw ; k_raw] = [W^DKV ; W^KR] h, then the append of those rows.
mla_status project_and_append(const mla_config* c, bool bf16, const mla_kv_cache* k, const mla_weights* w,
                              const void* h, int32_t B, int32_t L, int32_t start_pos, float* rope_cs,
                              float* kv_raw, hipStream_t st) {
  const int64_t T = (int64_t)B * L;
  const int row = c->d_c + c->d_rope;
  // with a table (prefill: q^R's RoPE reads it too) the append takes its
  // angles from it; without, the append forms them itself
  if (rope_cs) MLA_HIP(launch_rope_table(rope_cs, L, start_pos, c->d_rope, rope_params(c), st));
  GemmArgs g = gemm(h, c->d_model, 0, w->w_dkv, c->d_model, 0, kv_raw, row, 0, (int)T, row, c->d_model, 1, false,
                    false);
  g.B2 = w->w_kr;
  g.n_split = c->d_c;
  bool sk = false;
  if (const int G = kv_sk_groups(c, bf16, T)) {
    g.sk_wgs = G;
    g.sk_pstride = T * row;
    const hipError_t e = launch_gemm_bf16_streamk(g, st);
    if (e == hipSuccess)
      sk = true;
    else if (e != hipErrorNotSupported)
      return MLA_ERR_HIP;
    g.sk_wgs = 0;
  }
  if (!sk && launch_gemm(bf16, g, st) != MLA_OK) return MLA_ERR_HIP;
  AppendArgs a{};
  a.ckv = kv_raw; a.ld_ckv = row;
  a.kr = kv_raw + c->d_c; a.ld_kr = row;
  a.g_kv = w->g_kv;
  a.seq_idx = nullptr; a.pos = nullptr;
  a.n = (int32_t)T; a.n_seqs = B; a.L = L; a.start_pos = start_pos;
  a.in_f32 = 1;
  a.part_stride = sk ? T * row : 0;
  a.sk_wgs = sk ? kv_sk_groups(c, bf16, T) : 0;
  a.sk_nk = c->d_model / GEMM_SK_BK;
  a.rope_cs = rope_cs;
  a.pool = k->pool; a.num_pages = k->num_pages;
  a.block_table = k->block_table; a.max_pages = k->max_pages_per_seq; a.page_size = c->page_size;
  a.err_flags = k->err_flags;
  a.d_c = c->d_c; a.d_rope = c->d_rope;
  a.eps = c->rms_eps; a.rope = rope_params(c);
  a.bf16_cache = bf16 ? 1 : 0;
  a.fp8_cache = c->kv_fp8;
  MLA_HIP(launch_append(a, st));
  return MLA_OK;
}

AttnArgs attn_args(const mla_config* c, const mla_kv_cache* k, const void* q_lat, int32_t ld_q, const void* q_rope,
                   int32_t ld_r, const int32_t* kv_lens, int32_t uniform_kv, int32_t max_kv, int32_t B, int32_t s_q) {
  AttnArgs a{};
  a.q_lat = q_lat;
  a.ld_q = ld_q;
  a.q_rope = q_rope;
  a.ld_r = ld_r;
  a.pool = k->pool;
  a.fp8 = c->kv_fp8;
  a.block_table = k->block_table;
  a.num_pages = k->num_pages;
  a.max_pages = k->max_pages_per_seq;
  a.page_size = c->page_size;
  a.err_flags = k->err_flags;
  a.kv_lens = kv_lens;
  a.uniform_kv = uniform_kv;
  a.max_kv = max_kv;
  a.B = B;
  a.s_q = s_q;
  a.H = c->n_heads;
  a.d_c = c->d_c;
  a.d_rope = c->d_rope;
  a.scale = logit_scale(c);
  return a;
}

// The plan / split-partial fields of an attention call.
void set_plan(AttnArgs& a, int32_t* plan, int64_t max_items, void* part_o, float* part_ml, void* o_lat) {
  a.o_lat = o_lat;
  a.plan = plan;
  a.max_items = (int32_t)max_items;
  a.part_o = part_o;
  a.part_ml = part_ml;
}

// Attention + merge + W^UV for rows whose absorbed queries are in q_abs (a
// carries the plan fields; plan_built: the plan is already on the stream).
mla_status attend(const mla_config* c, bool bf16, const AttnArgs& a, int32_t target, bool plan_built,
                  bool need_merge, const void* w_uv, void* out, hipStream_t st, void* ev0, void* ev1) {
  const int64_t rows = (int64_t)a.B * a.s_q;
  const void* o_lat = a.o_lat;
  if (bf16) {
    if (!plan_built)
      MLA_HIP(launch_attn_plan(a, const_cast<int32_t*>(a.plan), target, MIN_CHUNK, max_chunk_keys(c) / 32 * 32, st));
    if (ev0) MLA_HIP(hipEventRecord((hipEvent_t)ev0, st));
    MLA_HIP(launch_attn_bf16(a, st));
    if (ev1) MLA_HIP(hipEventRecord((hipEvent_t)ev1, st));
    if (need_merge && rows <= MERGE_WUV_MAX_ROWS && c->d_head == 128) {
      // merge and W^UV in one pass
      MLA_HIP(launch_merge_wuv_bf16(a, w_uv, out, st));
      return MLA_OK;
    }
    if (need_merge) MLA_HIP(launch_merge_bf16(a, st));
  } else {
    if (ev0) MLA_HIP(hipEventRecord((hipEvent_t)ev0, st));
    MLA_HIP(launch_attn_f32(a, st));
    if (ev1) MLA_HIP(hipEventRecord((hipEvent_t)ev1, st));
  }
  // o[t, i, :] = W_i^UV o_lat[t, i, :]
  GemmArgs g = gemm(o_lat, (int64_t)c->n_heads * c->d_c, c->d_c, w_uv, c->d_c, (int64_t)c->d_head * c->d_c, out,
                    (int64_t)c->n_heads * c->d_head, c->d_head, (int)rows, c->d_head, c->d_c, c->n_heads, false, bf16);
  return launch_gemm(bf16, g, st);
}

// Steps (3) to (10) of the explicit form, after q^C and the raw q^R are in the
// workspace: RoPE of q^R, k^C = W^UK c and v^C = W^UV c for rows
// [0, start_pos + L) of every sequence, then causal attention.
mla_status prefill_explicit(const mla_config* c, const mla_kv_cache* k, const mla_weights* w, int32_t B, int32_t L,
                            int32_t start_pos, const PrefillWs& p, bool qr_done, void* out, hipStream_t st, void* ev0,
                            void* ev1) {
  const int T = B * L, H = c->n_heads, row = c->d_c + c->d_rope, kv_end = start_pos + L;
  const int nk = B * kv_end;
  if (!qr_done) MLA_HIP(launch_rope_heads(p.qr_raw, p.rope_cs, L, p.qr, c->d_rope, 0, T, H, c->d_rope, 1, st));
  GatherArgs g{};
  g.pool = k->pool; g.num_pages = k->num_pages;
  g.block_table = k->block_table; g.max_pages = k->max_pages_per_seq; g.page_size = c->page_size;
  g.B = B; g.kv_end = kv_end; g.row = row;
  g.fp8 = c->kv_fp8;
  g.err_flags = k->err_flags;
  g.out = p.kvg;
  MLA_HIP(launch_gather_rows(g, st));
  // k^C[j, i, :] = W_i^UK c_j and v^C[j, i, :] = W_i^UV c_j: [nk, d_c] x [H d_h, d_c]^T
  mla_status s;
  if ((s = launch_gemm(true, gemm(p.kvg, row, 0, w->w_uk, c->d_c, 0, p.kc, (int64_t)H * c->d_head, 0, nk,
                                  H * c->d_head, c->d_c, 1, false, true), st)) != MLA_OK)
    return s;
  if ((s = launch_gemm(true, gemm(p.kvg, row, 0, w->w_uv, c->d_c, 0, p.vc, (int64_t)H * c->d_head, 0, nk,
                                  H * c->d_head, c->d_c, 1, false, true), st)) != MLA_OK)
    return s;
  FaArgs a{};
  a.qc = p.qc; a.qr = p.qr;
  a.kc = p.kc; a.vc = p.vc;
  a.kr = (const unsigned char*)p.kvg + (size_t)c->d_c * 2;
  a.ld_kr = row;
  a.B = B; a.L = L; a.H = H; a.start_pos = start_pos; a.kv_end = kv_end;
  a.scale = logit_scale(c);
  a.out = out;
  if (ev0) MLA_HIP(hipEventRecord((hipEvent_t)ev0, st));
  MLA_HIP(launch_fa_bf16(a, st));
  if (ev1) MLA_HIP(hipEventRecord((hipEvent_t)ev1, st));
  return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

int64_t mla_cache_row_bytes(const mla_config* cfg) {
  bool bf16;
  if (check_cfg(cfg, &bf16) != MLA_OK) return -1;
  if (cfg->kv_fp8) return 656;
  return (int64_t)(cfg->d_c + cfg->d_rope) * (bf16 ? 2 : 4);
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, non-positive size or misaligned pointer";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape or dtype not implemented";
    case MLA_ERR_OUT_OF_RANGE: return "MLA_ERR_OUT_OF_RANGE: length exceeds the cache";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP launch or runtime call failed";
  }
  return "unknown mla_status";
}

mla_status mla_cache_append(const mla_config* cfg, const mla_kv_cache* cache, const void* ckv_raw,
                            const void* kr_raw, const void* g_kv, const int32_t* seq_idx, const int32_t* pos,
                            int32_t n, int32_t n_seqs, void* stream) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if ((s = check_cache(cfg, cache)) != MLA_OK) return s;
  if (n < 0 || n_seqs <= 0) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!ckv_raw || !kr_raw || !g_kv || !seq_idx || !pos) return MLA_ERR_INVALID_ARG;
  if (!aligned16(ckv_raw) || !aligned16(kr_raw) || !aligned16(g_kv)) return MLA_ERR_INVALID_ARG;
  AppendArgs a{};
  a.ckv = ckv_raw; a.ld_ckv = cfg->d_c;
  a.kr = kr_raw; a.ld_kr = cfg->d_rope;
  a.g_kv = g_kv;
  a.seq_idx = seq_idx; a.pos = pos;
  a.n = n; a.n_seqs = n_seqs; a.L = 1; a.start_pos = 0;
  a.in_f32 = bf16 ? 0 : 1;
  a.rope_cs = nullptr;
  a.pool = cache->pool; a.num_pages = cache->num_pages;
  a.block_table = cache->block_table; a.max_pages = cache->max_pages_per_seq; a.page_size = cfg->page_size;
  a.err_flags = cache->err_flags;
  a.d_c = cfg->d_c; a.d_rope = cfg->d_rope;
  a.eps = cfg->rms_eps; a.rope = rope_params(cfg);
  a.bf16_cache = bf16 ? 1 : 0;
  a.fp8_cache = cfg->kv_fp8;
  return launch_append(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_project_kv_workspace_size(const mla_config* cfg, int32_t B, int32_t L, size_t* bytes) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if (!bytes || B < 0 || L < 0) return MLA_ERR_INVALID_ARG;
  float *a, *b;
  *bytes = project_kv_layout(cfg, bf16, B, L, nullptr, &a, &b);
  return MLA_OK;
}

mla_status mla_project_kv(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w, const void* h,
                          int32_t B, int32_t L, int32_t start_pos, void* ws, size_t ws_bytes, void* stream) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if ((s = check_cache(cfg, cache)) != MLA_OK) return s;
  if (B < 0 || L < 0 || start_pos < 0) return MLA_ERR_INVALID_ARG;
  if (B == 0 || L == 0) return MLA_OK;
  if (!w || !w->w_dkv || !w->w_kr || !w->g_kv || !h || !ws) return MLA_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w->w_dkv) || !aligned16(w->w_kr) || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
  if (B > (1 << 20) || (int64_t)start_pos + L > (int64_t)cache->max_pages_per_seq * cfg->page_size)
    return MLA_ERR_OUT_OF_RANGE;
  float *rope_cs, *kv_raw;
  if (project_kv_layout(cfg, bf16, B, L, ws, &rope_cs, &kv_raw) > ws_bytes) return MLA_ERR_WORKSPACE;
  return project_and_append(cfg, bf16, cache, w, h, B, L, start_pos, nullptr, kv_raw, (hipStream_t)stream);
}

mla_status mla_prefill_workspace_size(const mla_config* cfg, int32_t B, int32_t L, int32_t start_pos,
                                      size_t* bytes) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if (!bytes || B < 0 || L < 0 || start_pos < 0) return MLA_ERR_INVALID_ARG;
  bool use_explicit;
  if ((s = prefill_form(cfg, bf16, L, start_pos, &use_explicit)) != MLA_OK) return s;
  prefill_layout(cfg, bf16, use_explicit, B, L, start_pos, nullptr, bytes);
  return MLA_OK;
}

mla_status mla_prefill(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w, const void* h,
                       int32_t B, int32_t L, int32_t start_pos, void* out, void* ws, size_t ws_bytes, void* stream) {
  return mla_prefill_profiled(cfg, cache, w, h, B, L, start_pos, out, ws, ws_bytes, stream, nullptr, nullptr);
}

mla_status mla_prefill_profiled(const mla_config* cfg, const mla_kv_cache* cache, const mla_weights* w,
                                const void* h, int32_t B, int32_t L, int32_t start_pos, void* out, void* ws,
                                size_t ws_bytes, void* stream, void* attn_start, void* attn_stop) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if ((s = check_cache(cfg, cache)) != MLA_OK) return s;
  if (B < 0 || L < 0 || start_pos < 0) return MLA_ERR_INVALID_ARG;
  if (B == 0 || L == 0) return MLA_OK;
  if (!w || !h || !out || !ws || !w->w_dq || !w->g_q || !w->w_uq || !w->w_qr || !w->w_dkv || !w->g_kv ||
      !w->w_kr || !w->w_uk || !w->w_uv)
    return MLA_ERR_INVALID_ARG;
  const void* ptrs[] = {h, out, ws, w->w_dq, w->w_uq, w->w_qr, w->w_dkv, w->w_kr, w->w_uk, w->w_uv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_INVALID_ARG;
  const int64_t kv_end = (int64_t)start_pos + L;
  if (kv_end > (int64_t)cache->max_pages_per_seq * cfg->page_size || kv_end > (1 << 30)) return MLA_ERR_OUT_OF_RANGE;
  if ((int64_t)B * L > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  bool use_explicit;
  if ((s = prefill_form(cfg, bf16, L, start_pos, &use_explicit)) != MLA_OK) return s;
  if (use_explicit && (int64_t)B * kv_end > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  size_t need;
  PrefillWs p = prefill_layout(cfg, bf16, use_explicit, B, L, start_pos, ws, &need);
  if (need > ws_bytes) return MLA_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int T = B * L, H = cfg->n_heads, row = cfg->d_c + cfg->d_rope;
  // steps (5), (7): cached latents, then the append
  if ((s = project_and_append(cfg, bf16, cache, w, h, B, L, start_pos, p.rope_cs, p.kv_raw, st)) != MLA_OK) return s;
  // step (1): c^Q = RMSNorm(W^DQ h)
  if ((s = launch_gemm(bf16, gemm(h, cfg->d_model, 0, w->w_dq, cfg->d_model, 0, p.cq_raw, cfg->d_cq, 0, T,
                                  cfg->d_cq, cfg->d_model, 1, false, false), st)) != MLA_OK)
    return s;
  MLA_HIP(launch_rmsnorm(p.cq_raw, cfg->d_cq, w->g_q, p.cq, cfg->d_cq, T, cfg->d_cq, cfg->rms_eps, bf16, st));
  // step (2): q^C = W^UQ c^Q
  if ((s = launch_gemm(bf16, gemm(p.cq, cfg->d_cq, 0, w->w_uq, cfg->d_cq, 0, p.qc, (int64_t)H * cfg->d_head, 0, T,
                                  H * cfg->d_head, cfg->d_cq, 1, false, bf16), st)) != MLA_OK)
    return s;
  // step (3): q^R = RoPE(W^QR c^Q).  Explicit form: the rotation runs in the
  // GEMM's output stage where that form applies; otherwise the GEMM writes fp32
  // and a separate pass rotates (into the absorbed query for that form).
  bool qr_done = false;
  if (p.use_explicit) {
    GemmArgs gq = gemm(p.cq, cfg->d_cq, 0, w->w_qr, cfg->d_cq, 0, p.qr, (int64_t)H * cfg->d_rope, 0, T,
                       H * cfg->d_rope, cfg->d_cq, 1, false, true);
    gq.rope_cs = p.rope_cs; gq.rope_rows = L; gq.rope_d = cfg->d_rope;
    const hipError_t e = launch_gemm_bf16_rope(gq, st);
    if (e == hipSuccess)
      qr_done = true;
    else if (e != hipErrorNotSupported)
      return MLA_ERR_HIP;
  }
  if (!qr_done && (s = launch_gemm(bf16, gemm(p.cq, cfg->d_cq, 0, w->w_qr, cfg->d_cq, 0, p.qr_raw,
                                              (int64_t)H * cfg->d_rope, 0, T, H * cfg->d_rope, cfg->d_cq, 1, false,
                                              false), st)) != MLA_OK)
    return s;
  if (p.use_explicit)
    return prefill_explicit(cfg, cache, w, B, L, start_pos, p, qr_done, out, st, attn_start, attn_stop);
  MLA_HIP(launch_rope_heads(p.qr_raw, p.rope_cs, L, p.q_abs, row, cfg->d_c, T, H, cfg->d_rope, bf16, st));
  // absorption: q_lat_i = W_i^UK^T q^C_i  (batched over heads, W_i^UK given [d_h, d_c])
  if ((s = launch_gemm(bf16, gemm(p.qc, (int64_t)H * cfg->d_head, cfg->d_head, w->w_uk, cfg->d_c,
                                  (int64_t)cfg->d_head * cfg->d_c, p.q_abs, (int64_t)H * row, row, T, cfg->d_c,
                                  cfg->d_head, H, true, bf16), st)) != MLA_OK)
    return s;
  // step (10) in absorbed form over rows [0, start_pos + t]
  const size_t e = bf16 ? 2 : 4;
  AttnArgs a = attn_args(cfg, cache, p.q_abs, row, (const unsigned char*)p.q_abs + cfg->d_c * e, row, nullptr,
                         (int32_t)kv_end, (int32_t)kv_end, B, L);
  a.longest_first = 1;
  set_plan(a, p.plan, p.max_items, p.part_o, p.part_ml, p.o_lat);
  return attend(cfg, bf16, a, 0, false, p.split, w->w_uv, out, st, attn_start, attn_stop);
}

mla_status mla_decode_workspace_size(const mla_config* cfg, int32_t B, int32_t s_q, int32_t max_kv_len,
                                     size_t* bytes) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if (!bytes || B < 0 || s_q < 0 || max_kv_len < 0) return MLA_ERR_INVALID_ARG;
  decode_layout(cfg, bf16, B, s_q, max_kv_len, nullptr, bytes);
  return MLA_OK;
}

int32_t mla_decode_num_splits(const mla_config* cfg, int32_t B, int32_t s_q, int32_t max_kv_len) {
  bool bf16;
  if (check_cfg(cfg, &bf16) != MLA_OK || B <= 0 || s_q <= 0 || max_kv_len <= 0) return 0;
  if (!bf16) return 1;
  return (int32_t)max_plan_items(cfg, (int64_t)B * s_q, max_kv_len, DECODE_TARGET_ITEMS);
}

mla_status mla_decode(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens, int32_t max_kv_len,
                      int32_t B, int32_t s_q, const void* q_nope, const void* q_pe, const void* w_uk,
                      const void* w_uv, void* out, void* ws, size_t ws_bytes, void* stream) {
  return mla_decode_profiled(cfg, cache, kv_lens, max_kv_len, B, s_q, q_nope, q_pe, w_uk, w_uv, out, ws, ws_bytes,
                             stream, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Checks of mla_decode's arguments other than the workspace; *empty when
// there is nothing to do (B == 0 or s_q == 0).
mla_status decode_check(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens, int32_t max_kv_len,
                        int32_t B, int32_t s_q, const void* q_nope, const void* q_pe, const void* w_uk,
                        const void* w_uv, void* out, bool* bf16, bool* empty) {
  mla_status s = check_cfg(cfg, bf16);
  if (s != MLA_OK) return s;
  if ((s = check_cache(cfg, cache)) != MLA_OK) return s;
  if (B < 0 || s_q < 0) return MLA_ERR_INVALID_ARG;
  *empty = B == 0 || s_q == 0;
  if (*empty) return MLA_OK;
  if (!kv_lens || !q_nope || !q_pe || !w_uk || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  const void* ptrs[] = {q_nope, q_pe, w_uk, w_uv, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_INVALID_ARG;
  if (max_kv_len < s_q) return MLA_ERR_INVALID_ARG;
  if ((int64_t)max_kv_len > (int64_t)cache->max_pages_per_seq * cfg->page_size || max_kv_len > (1 << 30))
    return MLA_ERR_OUT_OF_RANGE;
  if ((int64_t)B * s_q > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The decode launches over a carved workspace.
mla_status decode_run(const mla_config* cfg, bool bf16, const mla_kv_cache* cache, const int32_t* kv_lens,
                      int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope, const void* q_pe,
                      const void* w_uk, const void* w_uv, void* out, const DecodeWs& d, hipStream_t st,
                      void* attn_start, void* attn_stop) {
  mla_status s;
  const int rows = B * s_q, H = cfg->n_heads;
  AttnArgs a = attn_args(cfg, cache, d.q_lat, cfg->d_c, q_pe, cfg->d_rope, kv_lens, 0, max_kv_len, B, s_q);
  a.longest_first = 0;
  set_plan(a, d.plan, d.max_items, d.part_o, d.part_ml, d.o_lat);
  // absorption: q_lat[t, i, :] = W_i^UK^T q^C[t, i]  (q^R is read from q_pe
  // directly); the split plan is built by one extra workgroup of that launch
  const GemmArgs absorb = gemm(q_nope, (int64_t)H * cfg->d_head, cfg->d_head, w_uk, cfg->d_c,
                               (int64_t)cfg->d_head * cfg->d_c, d.q_lat, (int64_t)H * cfg->d_c, cfg->d_c, rows,
                               cfg->d_c, cfg->d_head, H, true, bf16);
  if (bf16) {
    PlanJob pj{a, d.plan, DECODE_TARGET_ITEMS, MIN_CHUNK, max_chunk_keys(cfg) / 32 * 32};
    MLA_HIP(launch_gemm_bf16_plan(absorb, pj, st));
  } else if ((s = launch_gemm(bf16, absorb, st)) != MLA_OK) {
    return s;
  }
  return attend(cfg, bf16, a, DECODE_TARGET_ITEMS, true, true, w_uv, out, st, attn_start, attn_stop);
}

// ---- decode without allocation: the workspace is a scratch array in each
// GPU's memory, found once per device with hipGetSymbolAddress (in host code
// the array's name is not a device address).
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES];

}  // namespace

static __device__ __align__(256) unsigned char scratch[MLA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

mla_status scratch_of_device(hipStream_t st, void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (st) {  // the stream must belong to the current device
    hipDevice_t sd;
    if (hipStreamGetDevice(st, &sd) != hipSuccess) return MLA_ERR_HIP;
    if ((int)sd != dev) return MLA_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= MAX_DEVICES) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MLA_ERR_HIP;
    g_scratch[dev] = q;
  }
  *p = g_scratch[dev];
  return MLA_OK;
}

// The scratch layout for these sizes: the usual decode workspace, with fewer
// split slots when the usual bound does not fit (the plan then makes fewer,
// longer chunks of ragged batches).  MLA_ERR_WORKSPACE when even the fewest
// slots the plan can work with do not fit.
mla_status noalloc_layout(const mla_config* cfg, bool bf16, int32_t B, int32_t s_q, int32_t max_kv, void* base,
                          DecodeWs* d) {
  const size_t cap = MLA_DECODE_NOALLOC_SCRATCH_BYTES;
  size_t need;
  *d = decode_layout(cfg, bf16, B, s_q, max_kv, base, &need);
  if (need <= cap) return MLA_OK;
  if (!bf16) return MLA_ERR_WORKSPACE;
  const int64_t rows = (int64_t)B * s_q;
  // slots the plan needs at least: every row one item (and 7 for the XCD
  // runs), and every row cut at the chunk cap
  const int64_t least = std::max(rows + 8, rows * ceil_div(max_kv, max_chunk_keys(cfg)) + 7);
  const size_t per_item = (size_t)cfg->n_heads * cfg->d_c * 2 + (size_t)cfg->n_heads * 2 * 4 + 16;
  int64_t items = d->max_items - (int64_t)((need - cap + per_item - 1) / per_item);
  items = items / 8 * 8;
  for (; items >= least; items -= 8) {
    *d = decode_layout(cfg, bf16, B, s_q, max_kv, base, &need, items);
    if (need <= cap) return MLA_OK;
  }
  return MLA_ERR_WORKSPACE;
}

}  // namespace

extern "C" {

mla_status mla_decode_profiled(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens,
                               int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope, const void* q_pe,
                               const void* w_uk, const void* w_uv, void* out, void* ws, size_t ws_bytes,
                               void* stream, void* attn_start, void* attn_stop) {
  bool bf16, empty;
  mla_status s = decode_check(cfg, cache, kv_lens, max_kv_len, B, s_q, q_nope, q_pe, w_uk, w_uv, out, &bf16, &empty);
  if (s != MLA_OK || empty) return s;
  if (!ws || !aligned16(ws)) return MLA_ERR_INVALID_ARG;
  size_t need;
  DecodeWs d = decode_layout(cfg, bf16, B, s_q, max_kv_len, ws, &need);
  if (need > ws_bytes) return MLA_ERR_WORKSPACE;
  return decode_run(cfg, bf16, cache, kv_lens, max_kv_len, B, s_q, q_nope, q_pe, w_uk, w_uv, out, d,
                    (hipStream_t)stream, attn_start, attn_stop);
}

mla_status mla_decode_noalloc(const mla_config* cfg, const mla_kv_cache* cache, const int32_t* kv_lens,
                              int32_t max_kv_len, int32_t B, int32_t s_q, const void* q_nope, const void* q_pe,
                              const void* w_uk, const void* w_uv, void* out, void* stream) {
  bool bf16, empty;
  mla_status s = decode_check(cfg, cache, kv_lens, max_kv_len, B, s_q, q_nope, q_pe, w_uk, w_uv, out, &bf16, &empty);
  if (s != MLA_OK || empty) return s;
  DecodeWs d;
  if ((s = noalloc_layout(cfg, bf16, B, s_q, max_kv_len, nullptr, &d)) != MLA_OK) return s;  // sizes first
  void* base;
  if ((s = scratch_of_device((hipStream_t)stream, &base)) != MLA_OK) return s;
  if ((s = noalloc_layout(cfg, bf16, B, s_q, max_kv_len, base, &d)) != MLA_OK) return s;
  return decode_run(cfg, bf16, cache, kv_lens, max_kv_len, B, s_q, q_nope, q_pe, w_uk, w_uv, out, d,
                    (hipStream_t)stream, nullptr, nullptr);
}

// Split of the output projection's reduction: enough workgroups to stream W^O
// at full bandwidth when T is small, each slice at least 512 wide.
int32_t out_proj_splits(const mla_config* c, bool bf16, int32_t T, int32_t width) {
  if (!bf16) return 1;
  const int64_t tiles = ceil_div(T, 128) * ceil_div(c->d_model, 128);
  int64_t s = ceil_div(768, tiles);
  s = s < width / 512 ? s : width / 512;
  while (s > 1 && width % (s * 64) != 0) --s;
  return s > 1 ? (int32_t)s : 1;
}

mla_status mla_output_projection_workspace_size(const mla_config* cfg, int32_t T, int32_t width, size_t* bytes) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if (!bytes || T < 0 || width <= 0) return MLA_ERR_INVALID_ARG;
  const int32_t S = out_proj_splits(cfg, bf16, T, width);
  *bytes = S > 1 ? (size_t)S * T * cfg->d_model * 4 : 0;
  return MLA_OK;
}

mla_status mla_output_projection(const mla_config* cfg, const void* x, int32_t width, const void* w_o, void* u,
                                 int32_t T, void* ws, size_t ws_bytes, void* stream) {
  bool bf16;
  mla_status s = check_cfg(cfg, &bf16);
  if (s != MLA_OK) return s;
  if (T < 0 || width <= 0) return MLA_ERR_INVALID_ARG;
  if (T == 0) return MLA_OK;
  if (!x || !w_o || !u || !aligned16(x) || !aligned16(w_o) || !aligned16(u)) return MLA_ERR_INVALID_ARG;
  if (width % 64 != 0 || cfg->d_model % 8 != 0) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)T > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  const int32_t S = out_proj_splits(cfg, bf16, T, width);
  hipStream_t st = (hipStream_t)stream;
  const int d = cfg->d_model;
  if (S == 1)  // u[t, n] = sum_k x[t, k] W^O[n, k]
    return launch_gemm(bf16, gemm(x, width, 0, w_o, width, 0, u, d, 0, T, d, width, 1, false, bf16), st);
  if (!ws || !aligned16(ws) || (size_t)S * T * d * 4 > ws_bytes) return MLA_ERR_WORKSPACE;
  // slice z of the reduction: columns [z*Ks, (z+1)*Ks) of x and W^O into fp32 partial z
  const int32_t Ks = width / S;
  if ((s = launch_gemm(true, gemm(x, width, Ks, w_o, width, Ks, ws, d, (int64_t)T * d, T, d, Ks, S, false, false),
                       st)) != MLA_OK)
    return s;
  MLA_HIP(launch_sum_partials((const float*)ws, S, (int64_t)T * d, u, 1, st));
  return MLA_OK;
}

}  // extern "C"
