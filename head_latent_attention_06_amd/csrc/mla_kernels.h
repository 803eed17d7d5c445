// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Latent attention of query rows over a sequence's paged cache.  Query row
// r = b*s_q + s sits at position kv_len(b) - s_q + s and sees cache rows
// [0, that position].  A device work plan cuts every row's visible keys into
// chunks of `chunk` keys; each (chunk, head group of 128) is one workgroup.
//
// Plan layout (int32, device): [0] n_items, [1] chunk, [2 + r] first item of
// row r for r = 0 .. n_rows (row r owns items plan[2+r] .. plan[3+r]-1), then
// from plan_info_offset(n_rows) one int4 per workgroup of the attention grid,
// in launch order: {row, first key, end key, item << 1 | row has several items};
// entries past the last item have first key == end key.
__host__ __device__ inline int64_t plan_info_offset(int64_t n_rows) { return (n_rows + 3 + 3) / 4 * 4; }
__host__ __device__ inline int64_t plan_ints(int64_t n_rows, int64_t max_items) {
  return plan_info_offset(n_rows) + 4 * max_items;
}

struct AttnArgs {
  const void* q_lat;          // [n_rows, H, ld_q]: first d_c = W_i^UK^T q^C_i
  const void* q_rope;         // [n_rows, H, ld_r]: first d_rope = q^R_i (rotated)
  int32_t ld_q, ld_r;
  const void* pool;           // [num_pages, page_size, d_c + d_rope] (fp8: 656-byte rows)
  int32_t fp8;                // FP8 cache rows (bf16 kernel only)
  const int32_t* block_table; // [B, max_pages]
  int64_t num_pages;
  int32_t max_pages, page_size;
  int32_t* err_flags;         // may be null
  const int32_t* kv_lens;     // [B] or null (then uniform_kv)
  int32_t uniform_kv, max_kv;
  int32_t B, s_q, H;
  int32_t d_c, d_rope;        // f32 path only; the bf16 kernel is fixed at 512 / 64
  const int32_t* plan;        // work plan (above)
  int32_t max_items;          // grid size (upper bound on plan[0])
  int32_t longest_first;      // run items in reverse order (rows with most keys last in the plan)
  float scale;                // softmax scale
  void* part_o;               // [max_items, H, d_c] bf16: chunk output / chunk sum
  float* part_ml;             // [max_items, H, 2]: chunk max (log2 domain), chunk sum
  void* o_lat;                // [n_rows, H, d_c]
};

// Plan: target_items > 0 balances chunks to about that many items (more for
// ragged batches); target_items == 0 uses max_chunk.  Chunks are multiples of
// 32 keys within [min_chunk, max_chunk].
hipError_t launch_attn_plan(const AttnArgs& a, int32_t* plan, int32_t target_items, int32_t min_chunk,
                            int32_t max_chunk, hipStream_t st);
hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_merge_bf16(const AttnArgs& a, hipStream_t st);
// merge (as launch_merge_bf16) fused with out[r, i, :] = W_i^UV o_lat[r, i, :]
// (d_head = 128); w_uv [H*128, 512], out [n_rows, H, 128] bf16
hipError_t launch_merge_wuv_bf16(const AttnArgs& a, const void* w_uv, void* out, hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st);

// Batched GEMM C[z][m][n] = sum_k A[z][m][k] * B[z](k, n) with fp32 accumulation.
// B(k, n) = B[n*ldb + k] (b_kn = false: weights stored [out, in]) or
//           B[k*ldb + n] (b_kn = true).  When B2 is set, rows n >= n_split of a
// [N, K] weight come from B2 (row n - n_split); b_kn must be false then.
struct GemmArgs {
  const void* A; int64_t lda, strideA;
  const void* B; int64_t ldb, strideB;
  const void* B2; int32_t n_split;  // rows n >= n_split of B come from B2 (row n - n_split), same ldb and strideB
  void* C; int64_t ldc, strideC;
  int32_t M, N, K, batch;
  int32_t b_kn;
  int32_t out_bf16;           // bf16 path: store C as bf16 (else fp32)
  // optional RoPE of the output (launch_gemm_bf16_rope): column n is dim
  // n % rope_d of a head, row m takes position row rope_cs row m % rope_rows
  // ([rows, rope_d/2, 2] cos/sin), interleaved pairs (2p, 2p+1)
  const float* rope_cs; int32_t rope_rows, rope_d;
  // stream-K form (launch_gemm_bf16_streamk): sk_wgs groups of workgroups
  // (one per GEMM_SK_BN column tile) share the (row tile, k slice) units of
  // GEMM_SK_BM-row tiles equally; partial p of a row tile goes to
  // C + p * sk_pstride (see gemm_sk_parts)
  int32_t sk_wgs; int64_t sk_pstride;
};

constexpr int GEMM_SK_BM = 256, GEMM_SK_BN = 192, GEMM_SK_BK = 32;

// Partial sums of row tile t of a stream-K product with U = row tiles *
// slices units over W groups: the runs holding the tile's first and last
// slice, and every run between, each wrote one partial.
__host__ __device__ inline int gemm_sk_parts(int64_t t, int64_t slices, int64_t U, int64_t W) {
  const int64_t first = ((t * slices + 1) * W - 1) / U;
  const int64_t last = ((t * slices + slices) * W - 1) / U;
  return (int)(last - first + 1);
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st);
// The stream-K form (fp32 output, batch 1); hipErrorNotSupported for shapes
// the large-tile kernel does not take.
hipError_t launch_gemm_bf16_streamk(const GemmArgs& g, hipStream_t st);
// The GEMM with RoPE applied to its bf16 output in the same kernel; returns
// hipErrorNotSupported (launching nothing) for shapes the fused form does not
// take, so the caller can run the GEMM and the rotation separately.
hipError_t launch_gemm_bf16_rope(const GemmArgs& g, hipStream_t st);

// A GEMM and, in one extra workgroup of the same launch, the attention work
// plan (launch_attn_plan's job); falls back to two launches for GEMM shapes
// without that form.
struct PlanJob {
  AttnArgs a;
  int32_t* plan;
  int32_t target_items, min_chunk, max_chunk;
};
hipError_t launch_gemm_bf16_plan(const GemmArgs& g, const PlanJob& p, hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t st);

// RoPE frequencies theta_p = base^(-2p/d_rope), or with yarn_s > 1 the YaRN
// ones: (1 - g) theta_p / yarn_s + g theta_p, g = clamp((r - alpha) / (beta -
// alpha), 0, 1), r = yarn_orig * theta_p / (2 pi).
struct RopeParams {
  float base;
  float yarn_s, yarn_alpha, yarn_beta;
  int32_t yarn_orig;
};

// Cache append: row i -> [RMSNorm(ckv[i]) ; RoPE(kr[i], pos)] into its page slot.
// seq_idx / pos may be null: then sequence = i / L and pos = start_pos + i % L.
struct AppendArgs {
  const void* ckv; int64_t ld_ckv;   // [n, d_c] rows, leading dimension in elements
  const void* kr;  int64_t ld_kr;    // [n, d_rope]
  const void* g_kv;
  const int32_t* seq_idx; const int32_t* pos;
  int32_t n, n_seqs, L, start_pos;
  int32_t in_f32;                    // ckv / kr are fp32 (else cfg dtype)
  int64_t part_stride;               // in_f32 with sk_wgs > 0: each value is the sum of the partial
                                     // products of a stream-K GEMM (part_stride elements apart) over
                                     // sk_wgs groups and sk_nk k slices (gemm_sk_parts); 0: one product
  int32_t sk_wgs, sk_nk;
  const float* rope_cs;              // optional [L, d_rope/2, 2] cos/sin for implicit positions
  void* pool; int64_t num_pages;
  const int32_t* block_table; int32_t max_pages, page_size;
  int32_t* err_flags;
  int32_t d_c, d_rope;
  float eps;
  RopeParams rope;
  int32_t bf16_cache;                // cache dtype is bf16 (else fp32)
  int32_t fp8_cache;                 // FP8 rows (656 bytes; d_c = 512, d_rope = 64)
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

// cos / sin of pos * theta_p for positions start_pos .. start_pos + L - 1,
// computed in double precision: out [L, d_rope/2, 2] fp32.
hipError_t launch_rope_table(float* out, int32_t L, int32_t start_pos, int32_t d_rope, const RopeParams& rp,
                             hipStream_t st);

// out[i] = sum_{z < S} p[z * n + i] (fp32 partials of a split-K GEMM) for
// i < n, stored in bf16 or fp32; 4 elements per thread (n % 4 == 0).
hipError_t launch_sum_partials(const float* p, int32_t S, int64_t n, void* out, int32_t bf16_out, hipStream_t st);

// RMSNorm of fp32 rows into the storage dtype: out[r] = x[r] / rms(x[r]) * g.
hipError_t launch_rmsnorm(const float* x, int64_t ldx, const void* g, void* out, int64_t ldo,
                          int32_t rows, int32_t width, float eps, int32_t bf16_io, hipStream_t st);

// RoPE of fp32 per-head rows x [T, H, d_rope] with a cos/sin table (row t uses
// table row t % table_rows) into out[t, h, out_off ...] of row stride ld_out
// per head.
hipError_t launch_rope_heads(const float* x, const float* cs, int32_t table_rows, void* out,
                             int64_t ld_out, int32_t out_off, int32_t T, int32_t H, int32_t d_rope,
                             int32_t bf16_out, hipStream_t st);

// Explicit-form causal prefill attention (d_qk = 128 + 64, d_v = 128, bf16).
// Query row t of sequence b sits at position start_pos + t and sees keys
// [0, start_pos + t] of that sequence.  Keys: row (b * kv_end + j) of kc / vc
// [*, H, 128] and of kr (first 64 of each row, row stride ld_kr elements).
struct FaArgs {
  const void* qc;             // [B * L, H, 128] q^C
  const void* qr;             // [B * L, H, 64] q^R (rotated)
  const void* kc;             // [B * kv_end, H, 128] k^C = W^UK c
  const void* vc;             // [B * kv_end, H, 128] v^C = W^UV c
  const void* kr;             // [B * kv_end, ld_kr]: first 64 = k^R (rotated)
  int32_t ld_kr;
  int32_t B, L, H, start_pos, kv_end;
  float scale;
  void* out;                  // [B * L, H, 128]
};
hipError_t launch_fa_bf16(const FaArgs& a, hipStream_t st);

// Rows [0, kv_end) of each sequence's paged cache, copied to
// out [B * kv_end, row] (bf16).  Missing pages give zero rows and set err_flags.
struct GatherArgs {
  const void* pool; int64_t num_pages;
  const int32_t* block_table; int32_t max_pages, page_size;
  int32_t B, kv_end, row;
  int32_t fp8;                // FP8 cache rows, decoded to bf16 (row = 576)
  int32_t* err_flags;
  void* out;
};
hipError_t launch_gather_rows(const GatherArgs& g, hipStream_t st);

}  // namespace mla
