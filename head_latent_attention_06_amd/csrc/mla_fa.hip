// Explicit-form causal prefill attention, and the gather of cached rows it
// reads.
//
// What is computed (notes page "【论文解读】DeepSeek-V3", section 一(一), the
// ten-step "完整计算过程" list): with k^C_{j,i} = W_i^UK c_j and
// v^C_{j,i} = W_i^UV c_j materialised per head (two GEMMs over the cached
// latents), the layer is ordinary causal multi-head attention
//     q_{t,i} = [q^C_{t,i} ; q^R_{t,i}],   k_{j,i} = [k^C_{j,i} ; k^R_j],
//     o_{t,i} = sum_{j <= t} softmax_j(q_{t,i} . k_{j,i} / sqrt(d_h + d_h^R)) v^C_{j,i}
// with d_qk = 192 and d_v = 128; the output is o directly (no W^UV after the
// sum).  This form needs 640 FLOP per (pair, head) where the absorbed form
// needs 2,176, at the price of the two GEMMs.
//
// Kernel design (gfx950): one workgroup = 4 waves = 256 queries of one head;
// wave w owns 64 queries (two 32-query MFMA blocks), so every key fragment
// read from LDS feeds two MFMAs.  64-key tiles of [k^C | k^R | v^C] move
// HBM -> LDS with direct-to-LDS buffer loads into a 3-stage ring (two tiles
// in flight).  Scores are computed transposed, S^T = K Q^T (keys on M,
// queries on N), so each lane holds the scores of one query and the
// exponentiated scores are the B operand of O^T = V^T P^T; V^T comes from
// transposing LDS reads of the value rows.  Online softmax in the log2
// domain with the lazy rescale of the latent kernel.
#include <math.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int FA_DH = 128, FA_DR = 64;        // d_h (q^C, k^C, v^C) and d_h^R
constexpr int FA_KT = 64;                     // keys per tile
constexpr int FA_QW = 64, FA_QG = 4 * FA_QW;  // queries per wave / per workgroup
// one LDS stage: k^C rows (256 B), k^R rows (128 B), v^C rows (256 B) of 64 keys
constexpr int FA_KC = 0, FA_KR = FA_KT * 256, FA_V = FA_KR + FA_KT * 128;
constexpr int FA_STAGE = FA_V + FA_KT * 256;  // 40960 bytes
constexpr int FA_NSTAGE = 3;                  // tile t in use, t+1 and t+2 in flight
constexpr int FA_DMA = 10;                    // 16-byte loads per thread per tile
constexpr float FA_LOG2E = 1.4426950408889634f;
constexpr float FA_SLACK = 8.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fa_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 fa_ld16(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// 16 bytes per lane from buffer offset voff into LDS at lds_addr + 16 * lane
// (asm: the compiler's wait-count pass would otherwise wait for it before
// every later LDS access; the kernel waits explicitly).
__device__ __forceinline__ void fa_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void fa_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short fa_s16x4;
__device__ __forceinline__ u32x2 fa_tr16(const unsigned char* p) {
  const fa_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) fa_s16x4*)(__attribute__((address_space(3))) unsigned char*)p);
  return __builtin_bit_cast(u32x2, v);
}
template <typename T>
__device__ __forceinline__ const T* fa_uniform(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// multiply the 16 AGPRs of one accumulator tuple by a per-lane factor
__device__ __forceinline__ void fa_scale_tuple(f32x16& t, float alpha) {
  float tmp;
#define FA_SCALE1(i) "v_accvgpr_read_b32 %16, %" #i "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %" #i ", %16\n\t"
  asm volatile(FA_SCALE1(0) FA_SCALE1(1) FA_SCALE1(2) FA_SCALE1(3) FA_SCALE1(4) FA_SCALE1(5) FA_SCALE1(6)
               FA_SCALE1(7) FA_SCALE1(8) FA_SCALE1(9) FA_SCALE1(10) FA_SCALE1(11) FA_SCALE1(12) FA_SCALE1(13)
               FA_SCALE1(14) FA_SCALE1(15)
               : "+a"(t[0]), "+a"(t[1]), "+a"(t[2]), "+a"(t[3]), "+a"(t[4]), "+a"(t[5]), "+a"(t[6]),
                 "+a"(t[7]), "+a"(t[8]), "+a"(t[9]), "+a"(t[10]), "+a"(t[11]), "+a"(t[12]), "+a"(t[13]),
                 "+a"(t[14]), "+a"(t[15]), "=&v"(tmp)
               : "v"(alpha));
#undef FA_SCALE1
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bf16_kernel(FaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[FA_NSTAGE * FA_STAGE];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  // work id -> (sequence, head, query group): the query groups of one head are
  // consecutive ids, run longest first, and consecutive ids share an XCD (and
  // its L2), so a head's k^C / v^C stream is read from HBM about once
  const int H = a.H;
  const int n_qg = (a.L + FA_QG - 1) / FA_QG;
  const int work = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int q0 = (n_qg - 1 - work % n_qg) * FA_QG;
  const int head = (work / n_qg) % H, b = work / n_qg / H;
  // keys [0, start_pos + last query of the workgroup]
  const int kv_hi = a.start_pos + min(q0 + FA_QG, a.L);
  const int ntiles = (kv_hi + FA_KT - 1) / FA_KT;
  const float scale_log2 = a.scale * FA_LOG2E;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  // ---- tile loads.  k^C / v^C rows of this head: H*128 bf16 apart; k^R rows:
  // ld_kr bf16 apart.  LDS chunk swizzles (16-byte chunk c of row r):
  //   k^C: c ^ (r & 15)        k^R: c ^ ((r >> 1) & 7)        v^C: c ^ 4 (r & 3)
  // make the QK fragment reads and the transposing V reads conflict-free.
  const int64_t krow_bytes = (int64_t)H * FA_DH * 2;
  int32_t dma_off[FA_DMA];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // k^C and v^C: instructions 4i + wave of 16
    const int P = (4 * i + wave) * 64 + lane, r = P >> 4, s = P & 15;
    dma_off[i] = (int32_t)(r * krow_bytes + ((s ^ (r & 15)) * 16));
    dma_off[6 + i] = (int32_t)(r * krow_bytes + ((s ^ (4 * (r & 3))) * 16));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // k^R: instructions 4i + wave of 8
    const int P = (4 * i + wave) * 64 + lane, r = P >> 3, s = P & 7;
    dma_off[4 + i] = r * (a.ld_kr * 2) + ((s ^ ((r >> 1) & 7)) * 16);
  }
  const int64_t key_base = (int64_t)b * a.kv_end;
  auto issue_tile = [&](int t) {  // tile t (possibly past the end: empty resources)
    const int kb0 = t * FA_KT;
    const int rows = max(0, min(FA_KT, kv_hi - kb0));
    const bf16* kc = fa_uniform((const bf16*)a.kc + (key_base + kb0) * H * FA_DH + head * FA_DH);
    const bf16* vc = fa_uniform((const bf16*)a.vc + (key_base + kb0) * H * FA_DH + head * FA_DH);
    const bf16* kr = fa_uniform((const bf16*)a.kr + (key_base + kb0) * a.ld_kr);
    const int32_t nb_kv = __builtin_amdgcn_readfirstlane(rows > 0 ? (int32_t)((rows - 1) * krow_bytes + FA_DH * 2) : 0);
    const int32_t nb_r = __builtin_amdgcn_readfirstlane(rows > 0 ? (rows - 1) * a.ld_kr * 2 + FA_DR * 2 : 0);
    const __amdgpu_buffer_rsrc_t rkc = fa_rsrc(kc, nb_kv), rvc = fa_rsrc(vc, nb_kv), rkr = fa_rsrc(kr, nb_r);
    const uint32_t st = __builtin_amdgcn_readfirstlane(smem_addr + (t % FA_NSTAGE) * FA_STAGE);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa_dma16(rkc, st + FA_KC + (4 * i + wave) * 1024, dma_off[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) fa_dma16(rkr, st + FA_KR + (4 * i + wave) * 1024, dma_off[4 + i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa_dma16(rvc, st + FA_V + (4 * i + wave) * 1024, dma_off[6 + i]);
  };
  issue_tile(0);
  issue_tile(1);

  // ---- Q^T fragments (B operand of S^T = K Q^T): query block qb (32 queries),
  // k step s covers dims 16s .. 16s+15 (s < 8: q^C, s >= 8: q^R).  Queries past
  // L load as zero.
  u32x4 qf[2][12];
  {
    const int qw0 = q0 + FA_QW * wave;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int t0 = qw0 + 32 * qb;
      const int nq = max(0, min(32, a.L - t0));
      const int64_t row0 = (int64_t)b * a.L + t0;
      const __amdgpu_buffer_rsrc_t rq = fa_rsrc(fa_uniform((const bf16*)a.qc + row0 * H * FA_DH + head * FA_DH),
                                                nq > 0 ? (int32_t)((nq - 1) * krow_bytes + FA_DH * 2) : 0);
      const __amdgpu_buffer_rsrc_t rr =
          fa_rsrc(fa_uniform((const bf16*)a.qr + row0 * H * FA_DR + head * FA_DR),
                  nq > 0 ? (nq - 1) * H * FA_DR * 2 + FA_DR * 2 : 0);
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[qb][s] = fa_ld16(rq, (int32_t)(l32 * krow_bytes) + 32 * s + 16 * hi);
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[qb][8 + s] = fa_ld16(rr, l32 * H * FA_DR * 2 + 32 * s + 16 * hi);
    }
  }
  // the queries (and tile 0) are waited for here, not inside the tile loop
  asm volatile("" ::"v"(qf[0][0]), "v"(qf[0][1]), "v"(qf[0][2]), "v"(qf[0][3]), "v"(qf[0][4]), "v"(qf[0][5]),
               "v"(qf[0][6]), "v"(qf[0][7]), "v"(qf[0][8]), "v"(qf[0][9]), "v"(qf[0][10]), "v"(qf[0][11]));
  asm volatile("" ::"v"(qf[1][0]), "v"(qf[1][1]), "v"(qf[1][2]), "v"(qf[1][3]), "v"(qf[1][4]), "v"(qf[1][5]),
               "v"(qf[1][6]), "v"(qf[1][7]), "v"(qf[1][8]), "v"(qf[1][9]), "v"(qf[1][10]), "v"(qf[1][11]));

  // per-lane LDS offsets.  QK A operand (key row 32 kb + l32, chunk 2s + hi):
  int kc_off[8], kr_off[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) kc_off[s] = FA_KC + l32 * 256 + (((2 * s + hi) ^ (l32 & 15)) * 16);
#pragma unroll
  for (int s = 0; s < 4; ++s) kr_off[s] = FA_KR + l32 * 128 + (((2 * s + hi) ^ ((l32 >> 1) & 7)) * 16);
  // V^T A operand via transposing reads: for key step ks (16 keys), read r
  // (keys 16 ks + 8 r + 4 hi + jl/4), dim block d: chunk 4 d + 2 g1 + (jl&3)/2
  // of the row, half jl & 1.
  const int g1 = (lane >> 4) & 1, jl = lane & 15, rl = 4 * hi + (jl >> 2);
  int v_off[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    v_off[d] = FA_V + rl * 256 + ((4 * (d ^ (rl & 3)) + 2 * g1 + ((jl & 3) >> 1)) * 16) + 8 * (jl & 1);

  f32x16 acc[4][2];  // O^T [dim block][query block], AGPRs
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][qb][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  const int qpos0 = a.start_pos + q0 + FA_QW * wave;  // position of the wave's first query

  // tiles whose keys are all after every query of this wave are only moved, not used
  const int nt_wave = min(ntiles, (qpos0 + FA_QW - 1) / FA_KT + 1);
  int t = 0;
  for (; t < nt_wave; ++t) {
    // tile t has landed once at most tile t+1's loads are outstanding
    fa_wait_vmcnt<FA_DMA>();
    __syncthreads();
    issue_tile(t + 2);  // into the stage that held tile t-1
    const unsigned char* S = smem + (t % FA_NSTAGE) * FA_STAGE;
    const int kb0 = t * FA_KT;

    // ---- S^T[key][query] = K Q^T: 2 key blocks x 2 query blocks x 12 k steps
    f32x16 sacc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < 12; ++s) {
        const u32x4 kf = *(const u32x4*)(S + (s < 8 ? kc_off[s] : kr_off[s - 8]) + kb * 32 * (s < 8 ? 256 : 128));
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (s == 0)
            asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sacc[kb][qb]) : "v"(kf), "v"(qf[qb][s]));
          else
            asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc[kb][qb]) : "v"(kf), "v"(qf[qb][s]));
        }
      }
    }
    // wait states before VALU reads the MFMA results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // ---- online softmax per query (log2 domain).  Lane holds, for query l32
    // of block qb, keys kb0 + 32 kb + 8 (i/4) + 4 hi + i%4.
    u32x4 pf[4][2];  // P^T fragments [key step][query block]
    if (kb0 + FA_KT - 1 > qpos0) {
      // a tile on the diagonal: key kb0 + 32 kb + 8 (i/4) + 4 hi + i%4 is
      // masked for query qpos0 + 32 qb + l32 when 8 (i/4) + i%4 exceeds thr
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int thr = qpos0 + 32 * qb + l32 - kb0 - 32 * kb - 4 * hi;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (8 * (i >> 2) + (i & 3) > thr) sacc[kb][qb][i] = -INFINITY;
        }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
      // a query's first tile always holds key 0, so mt is finite there and the
      // rescale below (alpha = 0) also initialises m_run
      const float mt = pair_max32(mx) * scale_log2;
      if (__any(mt > m_run[qb] + FA_SLACK)) {
        const float mn = fmaxf(m_run[qb], mt);
        const float alpha = exp2f(m_run[qb] - mn);
        l_run[qb] *= alpha;
        m_run[qb] = mn;
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int d = 0; d < 4; ++d) fa_scale_tuple(acc[d][qb], alpha);
        asm volatile("s_nop 4" ::: "memory");
      }
      const float neg_m = -m_run[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 8 * h2 + 2 * e;
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][i], scale_log2, neg_m));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][i + 1], scale_log2, neg_m));
            pf[2 * kb + h2][qb][e] = pack_bf16x2(e0, e1);
            l_run[qb] += e0 + e1;
          }
    }

    // ---- O^T[dim][query] += V^T[dim][key] P^T[key][query]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const unsigned char* vb = S + v_off[d] + ks * 16 * 256;
        const u32x2 lo = fa_tr16(vb), hv = fa_tr16(vb + 8 * 256);
        const u32x4 vf = {lo[0], lo[1], hv[0], hv[1]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[d][qb]) : "v"(vf), "v"(pf[ks][qb]));
      }
    }
  }
  for (; t < ntiles; ++t) {
    fa_wait_vmcnt<FA_DMA>();
    __syncthreads();
    issue_tile(t + 2);
  }
  fa_wait_vmcnt<0>();  // tiles past the end still write LDS: drain them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[2][0]),
                 "+a"(acc[2][1]), "+a"(acc[3][0]), "+a"(acc[3][1]));

  // ---- out[t][head][:] = O^T[:, t] / l.  Lane (l32, hi), tuple (d, qb),
  // register 4g + e: dim 32 d + 8 g + 4 hi + e of query 32 qb + l32; lanes l
  // and l + 32 trade halves (v_permlane32_swap) so each stores 8 whole dims.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = q0 + FA_QW * wave + 32 * qb + l32;
    const float inv = 1.f / pair_sum32(l_run[qb]);
    if (tq < a.L) {
      bf16* o = (bf16*)a.out + (((int64_t)b * a.L + tq) * H + head) * FA_DH;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          uint32_t own[2][2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int g = 2 * gp + k;
            own[k][0] = pack_bf16x2(acc[d][qb][4 * g] * inv, acc[d][qb][4 * g + 1] * inv);
            own[k][1] = pack_bf16x2(acc[d][qb][4 * g + 2] * inv, acc[d][qb][4 * g + 3] * inv);
          }
          u32x4 v;
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const auto r = __builtin_amdgcn_permlane32_swap(own[0][e], own[1][e], false, false);
            v[e] = r[0];
            v[2 + e] = r[1];
          }
          *reinterpret_cast<u32x4*>(o + 32 * d + 8 * (2 * gp + hi)) = v;
        }
    }
  }
}

// Rows [0, kv_end) of every sequence from the paged cache into a contiguous
// [B * kv_end, row] buffer (one 16-byte chunk per thread); a block-table entry
// outside the pool gives zeros and sets err_flags.
__global__ void gather_rows_kernel(GatherArgs g) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int cpr = g.row / 8;  // 16-byte chunks per row (bf16)
  const int64_t total = (int64_t)g.B * g.kv_end * cpr;
  if (idx >= total) return;
  const int c = (int)(idx % cpr);
  const int64_t rr = idx / cpr;
  const int b = (int)(rr / g.kv_end), j = (int)(rr % g.kv_end);
  const int pidx = j / g.page_size;
  u32x4 v = {0u, 0u, 0u, 0u};
  const int page = pidx < g.max_pages ? g.block_table[(int64_t)b * g.max_pages + pidx] : -1;
  if (page >= 0 && (int64_t)page < g.num_pages) {
    v = *reinterpret_cast<const u32x4*>((const bf16*)g.pool + ((int64_t)page * g.page_size + j % g.page_size) * g.row +
                                        8 * c);
  } else if (c == 0 && g.err_flags) {
    atomicOr(g.err_flags, 1);
  }
  *reinterpret_cast<u32x4*>((bf16*)g.out + rr * g.row + 8 * c) = v;
}

}  // namespace

hipError_t launch_fa_bf16(const FaArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.L <= 0 || a.H <= 0) return hipSuccess;
  const int64_t n = (int64_t)a.H * ((a.L + FA_QG - 1) / FA_QG) * a.B;
  if (n > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fa_bf16_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const GatherArgs& g, hipStream_t st) {
  const int64_t n = (int64_t)g.B * g.kv_end * (g.row / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace mla
