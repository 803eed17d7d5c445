// Split-context latent attention over the paged MLA cache, and the merge of
// the split partials.
//
// What is computed (notes page "【论文解读】DeepSeek-V3", section 一(一)3, the
// score split into a latent term and a RoPE term, and the 【思考】 passage on
// absorption): for query row (token, head i) with absorbed query
// Q = [q_lat ; q^R], q_lat = W_i^UK^T q^C_i,
//     s_j = (q_lat . c_j + q^R . k^R_j) * scale,   j <= query position,
//     o_lat = sum_j softmax(s)_j c_j                   (d_c = 512 values).
// W_i^UV is applied to o_lat afterwards by a GEMM.
//
// bf16 kernel design (gfx950, one workgroup = 4 waves = 128 heads of one token
// over one chunk of keys):
//  * Every head of a token reads the same 576-value cache rows, so a 32-key
//    tile is staged once in LDS and consumed by all 128 heads: the cache is
//    read from HBM exactly once per (token, chunk).
//  * Tiles move HBM -> LDS with direct-to-LDS buffer loads (no registers), three
//    tiles in flight over a ring of four LDS stages; keys past the visible
//    range fall outside the buffer resource and arrive as zeros.  The 16-byte
//    chunks of key row r sit at chunk index c ^ f(r), f(r) = (2r ^ r/4) & 7,
//    which keeps every LDS read pattern below free of bank conflicts.
//  * Wave w owns 32 heads.  Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 (keys on M, heads on N, 576 dims on K), with the
//    wave's Q^T fragments held in registers for the whole chunk.  In that
//    layout each lane holds 16 scores of ONE head, so the exponentiated scores
//    are already the B operand of O^T = V^T P^T (dims on M, heads on N, keys
//    on K) and the per-head softmax rescale of O^T is a per-lane scalar.
//  * V^T operands come straight from the row-major key tile through
//    ds_read_b64_tr_b16 (gfx950 transposing LDS read): within each 16-lane
//    group, output lane 4a+e receives element e of source lanes a, a+4, a+8,
//    a+12, so four source lanes pointing at four key rows give each output
//    lane four keys of one latent dim.
//  * Online softmax in the log2 domain; the running max is only raised when
//    a tile's max exceeds it by more than 8 (p <= 256 stays exact in fp32),
//    so the 256-register O^T accumulator (kept in AGPRs) is rescaled rarely.
//    Row max / sum across the two lane halves use v_permlane32_swap.
#include <math.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int DC = 512, DR = 64, ROW = DC + DR;  // cached row: c^KV then k^R
constexpr int TILE = 32;                         // keys per LDS tile
constexpr int RB = ROW * 2;                      // bytes per key row (1152, unpadded)
constexpr int STAGE = TILE * RB;                 // 36864 bytes per tile
constexpr int NSTAGE = 4, DEPTH = 3;             // LDS ring, tiles in flight
constexpr int DMA_PER_THREAD = STAGE / 16 / 256; // 9 16-byte loads per thread per tile
constexpr int WG_HEADS = 128;
constexpr int MAX_SPLIT_PAGES = 1536;            // page ids of one split, staged in LDS
constexpr int FLAG_BAD_PAGE = 1, FLAG_BAD_LEN = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;

__device__ __forceinline__ int kv_len_of(const AttnArgs& a, int b, bool& ok) {
  const int kv = a.kv_lens ? a.kv_lens[b] : a.uniform_kv;
  ok = kv >= a.s_q && kv <= a.max_kv;
  return kv;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int32_t bytes) {
  // Raw buffer (stride 0): loads at offsets >= bytes return zero.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// A pointer the compiler cannot prove wave-uniform, made uniform (SGPRs).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// LDS chunk swizzle of key row r (chunk c of the row sits at c ^ kswz(r))
__device__ __forceinline__ int kswz(int r) { return ((r << 1) ^ (r >> 2)) & 7; }
// 16 bytes per lane from buffer offset voff into LDS at lds_addr + 16 * lane.
// Issued in asm so the compiler's wait-count pass does not put a full vmcnt
// wait in front of every later LDS access; the kernel waits explicitly.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
__device__ __forceinline__ u32x2 lds_tr16(const unsigned char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) unsigned char*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Multiply the 16 AGPRs of one accumulator tuple by alpha, one register at a
// time through a single temporary VGPR (a compiler-written loop would pull the
// whole 256-register accumulator into VGPRs).
__device__ __forceinline__ void scale_acc_tuple(f32x16& t, float alpha) {
  float tmp;
#define MLA_SCALE1(i) "v_accvgpr_read_b32 %16, %" #i "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 %" #i ", %16\n\t"
  asm volatile(MLA_SCALE1(0) MLA_SCALE1(1) MLA_SCALE1(2) MLA_SCALE1(3) MLA_SCALE1(4) MLA_SCALE1(5)
               MLA_SCALE1(6) MLA_SCALE1(7) MLA_SCALE1(8) MLA_SCALE1(9) MLA_SCALE1(10) MLA_SCALE1(11)
               MLA_SCALE1(12) MLA_SCALE1(13) MLA_SCALE1(14) MLA_SCALE1(15)
               : "+a"(t[0]), "+a"(t[1]), "+a"(t[2]), "+a"(t[3]), "+a"(t[4]), "+a"(t[5]), "+a"(t[6]),
                 "+a"(t[7]), "+a"(t[8]), "+a"(t[9]), "+a"(t[10]), "+a"(t[11]), "+a"(t[12]), "+a"(t[13]),
                 "+a"(t[14]), "+a"(t[15]), "=&v"(tmp)
               : "v"(alpha));
#undef MLA_SCALE1
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[NSTAGE * STAGE];
  __shared__ int split_pages[MAX_SPLIT_PAGES];

  const int n_hg = (a.H + WG_HEADS - 1) / WG_HEADS;
  const int tid = threadIdx.x;
  const int n_items = a.plan[0];
  const int chunk = a.plan[1];
  // The grid is an upper bound on the plan's items, so blocks map to items in
  // launch order: the real items are then spread round-robin over all XCDs.
  // With longest_first they run in reverse plan order (rows with most keys are
  // planned last).
  const int bid = (int)blockIdx.x / n_hg, hg = (int)blockIdx.x % n_hg;
  if (bid >= n_items) return;
  const int w = a.longest_first ? n_items - 1 - bid : bid;
  const int n_rows = a.B * a.s_q;
  const int32_t* row_off = a.plan + 2;
  int lo = 0, hi_r = n_rows - 1;  // last row r with row_off[r] <= w
  while (lo < hi_r) {
    const int mid = (lo + hi_r + 1) >> 1;
    if (row_off[mid] <= w) lo = mid; else hi_r = mid - 1;
  }
  const int row = lo;
  const int split = w - row_off[row];
  const int n_split_row = row_off[row + 1] - row_off[row];
  const int b = row / a.s_q, sq = row % a.s_q;
  bool len_ok;
  const int kv = kv_len_of(a, b, len_ok);
  if (!len_ok) return;  // the plan gives such rows no items
  const int qpos = kv - a.s_q + sq;
  const int k0 = split * chunk;
  const int k1 = min(k0 + chunk, qpos + 1);
  if (k0 >= k1) return;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int head0 = hg * WG_HEADS + wave * 32;  // first head of this wave
  const bool wave_on = head0 < a.H;
  const int64_t qrow = row;
  const float scale_log2 = a.scale * LOG2E;

  // Q^T fragments: B operand of S^T = K Q^T; k step j covers dims 16j .. 16j+15
  // (j < 32: q_lat, j >= 32: q^R).  Heads past H load as zero.
  u32x4 qf[36];
  {
    const int nh = wave_on ? min(32, a.H - head0) : 0;
    const int64_t hrow = qrow * a.H + (wave_on ? head0 : 0);
    const __amdgpu_buffer_rsrc_t ql = make_rsrc((const bf16*)a.q_lat + hrow * a.ld_q, nh * a.ld_q * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc((const bf16*)a.q_rope + hrow * a.ld_r, nh * a.ld_r * 2);
    const int ol = l32 * a.ld_q * 2 + 16 * hi, orr = l32 * a.ld_r * 2 + 16 * hi;
#pragma unroll
    for (int j = 0; j < 32; ++j) qf[j] = buf_ld16(ql, ol + 32 * j);
#pragma unroll
    for (int j = 32; j < 36; ++j) qf[j] = buf_ld16(qr, orr + 32 * (j - 32));
  }

  f32x16 acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[x][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // ---- tile loads: wave w's instruction i covers LDS chunks (4i + w)*64 + lane
  // of the stage; LDS chunk P holds key row P / 72, row chunk (P % 72) ^ kswz(row).
  int32_t dma_off[DMA_PER_THREAD];
#pragma unroll
  for (int i = 0; i < DMA_PER_THREAD; ++i) {
    const int P = (4 * i + wave) * 64 + lane;
    const int r = P / 72, c = (P % 72) ^ kswz(P / 72);
    dma_off[i] = r * RB + c * 16;
  }
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  // The chunk's page ids (the block-table read is kept off the tile pipeline).
  const int pg_first = k0 / a.page_size;
  const int n_pages = (k1 - 1) / a.page_size - pg_first + 1;  // <= MAX_SPLIT_PAGES (host plan)
  for (int i = tid; i < n_pages; i += 256) {
    const int pidx = pg_first + i;
    split_pages[i] = pidx < a.max_pages ? bt[pidx] : -1;
  }
  __syncthreads();

  auto issue_tile = [&](int t) {
    const int kb = k0 + t * TILE;
    const int page = __builtin_amdgcn_readfirstlane(split_pages[kb / a.page_size - pg_first]);
    const bool pok = page >= 0 && (int64_t)page < a.num_pages;
    if (!pok && tid == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_PAGE);
    // rows of the tile are contiguous within one page; rows past k1 (and a
    // bad page) lie outside the resource and load as zeros
    const bf16* base = (const bf16*)a.pool + ((int64_t)(pok ? page : 0) * a.page_size + (kb % a.page_size)) * ROW;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(uniform_ptr(base), __builtin_amdgcn_readfirstlane(pok ? min(TILE, k1 - kb) * RB : 0));
    const uint32_t dst = __builtin_amdgcn_readfirstlane(smem_addr + (t % NSTAGE) * STAGE + wave * 1024);
#pragma unroll
    for (int i = 0; i < DMA_PER_THREAD; ++i) dma16(r, dst + i * 4096, dma_off[i]);
  };

  // QK operand (row l32, 16-byte chunk 2j + hi): per-lane offsets for j % 4,
  // plus 128 bytes per 4 k steps
  int qk_off[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) qk_off[jj] = l32 * RB + (((2 * jj + hi) ^ kswz(l32)) * 16);
  // V^T operand via transposing reads: for k step q, read r (keys 16q+8r+4hi+j/4)
  // and dim block blk: row = 16q + 8r + rl, chunk = 4blk + 2g1 + (j&3)/2, half j&1
  const int g1 = (lane >> 4) & 1, jl = lane & 15;
  const int rl = 4 * hi + (jl >> 2);
  int pv_off[2][2][2];  // [q][r][blk & 1]; + (blk >> 1) * 128 bytes
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int bo = 0; bo < 2; ++bo) {
        const int row = 16 * q + 8 * r + rl;
        const int c = 4 * bo + 2 * g1 + ((jl & 3) >> 1);
        pv_off[q][r][bo] = row * RB + ((c ^ kswz(row)) * 16) + 8 * (jl & 1);
      }

  const int ntiles = (k1 - k0 + TILE - 1) / TILE;
#pragma unroll
  for (int p = 0; p < DEPTH; ++p)
    if (p < ntiles) issue_tile(p);

  for (int t = 0; t < ntiles; ++t) {
    // this thread's loads of tile t are done once at most the later tiles'
    // loads are outstanding; the barrier then makes every thread's visible
    const int later = min(DEPTH - 1, ntiles - 1 - t);
    if (later >= 2) wait_vmcnt<2 * DMA_PER_THREAD>();
    else if (later == 1) wait_vmcnt<DMA_PER_THREAD>();
    else wait_vmcnt<0>();
    __syncthreads();
    // the stage of tile t + DEPTH last held tile t - 1, which every wave has
    // finished reading before the barrier
    if (t + DEPTH < ntiles) issue_tile(t + DEPTH);
    {  // waves past the last head compute on zero queries and store nothing
      const unsigned char* K = smem + (t % NSTAGE) * STAGE;
      const int kb = k0 + t * TILE;
      // ---- S^T[key][head] for the 32 keys of the tile, accumulated in VGPRs.
      // K fragments are read KW MFMAs ahead of use (one wave per SIMD: nothing
      // else hides the LDS latency); sched_barrier pins that order.
      constexpr int KW = 3;
      u32x4 kf[KW];
#pragma unroll
      for (int j = 0; j < KW - 1; ++j) kf[j] = *(const u32x4*)(K + qk_off[j & 3] + 128 * (j >> 2));
      f32x16 s;
#pragma unroll
      for (int j = 0; j < 36; ++j) {
        if (j + KW - 1 < 36) {
          const int jn = j + KW - 1;
          kf[jn % KW] = *(const u32x4*)(K + qk_off[jn & 3] + 128 * (jn >> 2));
        }
        if (j == 0) {
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(s) : "v"(kf[0]), "v"(qf[0]));
        } else if (j < 35) {
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(kf[j % KW]), "v"(qf[j]));
        } else {
          // the trailing wait states let VALU read the MFMA result
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
              : "+v"(s) : "v"(kf[j % KW]), "v"(qf[j]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // The first V^T fragments do not depend on the softmax: start them now.
      constexpr int VW = 3;  // V fragments in flight
      u32x4 vf[VW];
      auto load_v = [&](int m) {  // MFMA m: k step m >> 4, dim block m & 15
        const int q = m >> 4, blk = m & 15;
        const u32x2 lo = lds_tr16(K + pv_off[q][0][blk & 1] + 128 * (blk >> 1));
        const u32x2 hv = lds_tr16(K + pv_off[q][1][blk & 1] + 128 * (blk >> 1));
        return u32x4{lo[0], lo[1], hv[0], hv[1]};
      };
#pragma unroll
      for (int i = 0; i < VW - 1; ++i) vf[i] = load_v(i);
      __builtin_amdgcn_sched_barrier(0);

      // ---- online softmax (log2 domain); lane holds keys kb + 8*(i/4) + 4*hi + i%4 of head l32
      float mloc = -INFINITY;
      if (kb + TILE <= k1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] *= scale_log2;
          mloc = fmaxf(mloc, s[i]);
        }
      } else {
        const int rem = k1 - kb - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[i] = (8 * (i >> 2) + (i & 3) < rem) ? s[i] * scale_log2 : -INFINITY;
          mloc = fmaxf(mloc, s[i]);
        }
      }
      const float mt = pair_max32(mloc);
      if (m_run == -INFINITY) {
        m_run = mt;  // first tile: accumulator and sum are still zero
      } else if (__any(mt > m_run + RESCALE_SLACK)) {
        const float mn = fmaxf(m_run, mt);
        const float alpha = exp2f(m_run - mn);
        l_run *= alpha;
#pragma unroll
        for (int x = 0; x < 16; ++x) scale_acc_tuple(acc[x], alpha);
        m_run = mn;
      }
      // P^T fragments: scores 8q .. 8q+7 of this lane are the k slots of step q.
      u32x4 pf[2];
      float lsum = 0.f;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t pk = pack_bf16x2(exp2f(s[8 * q + 2 * d] - m_run), exp2f(s[8 * q + 2 * d + 1] - m_run));
          pf[q][d] = pk;
          lsum += bf16_lo(pk) + bf16_hi(pk);
        }
      l_run += lsum;
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T[dim][head] += V^T[dim][key] P^T[key][head]: 16 blocks of 32 dims per
      // k step, accumulated in AGPRs.  The wait states ahead of the first MFMA
      // cover VALU writes of the P fragments and of a rescaled accumulator.
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        if (m + VW - 1 < 32) vf[(m + VW - 1) % VW] = load_v(m + VW - 1);
        if (m == 0) {
          asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[0]) : "v"(vf[0]), "v"(pf[0]));
        } else {
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
              : "+a"(acc[m & 15]) : "v"(vf[m % VW]), "v"(pf[m >> 4]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!wave_on) return;
  // wait states before VALU reads of accumulators last written by an MFMA
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
                 "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]),
                 "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]));

  const float l_tot = pair_sum32(l_run);
  const int head = head0 + l32;
  if (head >= a.H) return;
  // normalised by this chunk's sum: the final output when the row is one
  // chunk, else a partial the merge combines with weights 2^(m - m*) * l
  const float inv = 1.f / l_tot;
  bf16* o = (n_split_row == 1 ? (bf16*)a.o_lat + (qrow * a.H + head) * DC
                              : (bf16*)a.part_o + ((int64_t)w * a.H + head) * DC) + 4 * hi;
#pragma unroll
  for (int blk = 0; blk < 16; ++blk)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 v;
      v[0] = pack_bf16x2(acc[blk][4 * q4] * inv, acc[blk][4 * q4 + 1] * inv);
      v[1] = pack_bf16x2(acc[blk][4 * q4 + 2] * inv, acc[blk][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2*>(o + 32 * blk + 8 * q4) = v;
    }
  if (n_split_row > 1 && hi == 0) {
    const int64_t slot = (int64_t)w * a.H + head;
    a.part_ml[slot * 2] = m_run;
    a.part_ml[slot * 2 + 1] = l_tot;
  }
}

// Merge of split partials o_k = acc_k / l_k (m_k in the log2 domain):
//   o_lat = sum_k 2^(m_k - m*) l_k o_k / sum_k 2^(m_k - m*) l_k,  m* = max_k m_k.
// Rows cut into a single chunk were written by the attention kernel; rows
// with no chunk (invalid length) are written as zero.
__global__ __launch_bounds__(128) void merge_bf16_kernel(AttnArgs a) {
  const int head = blockIdx.x % a.H;
  const int64_t row = blockIdx.x / a.H;
  const int t = threadIdx.x;
  const int32_t* row_off = a.plan + 2;
  const int i0 = row_off[row], n = row_off[row + 1] - i0;
  if (n == 1) return;
  bf16* o = (bf16*)a.o_lat + (row * a.H + head) * DC + 4 * t;
  u32x2 outv = {0u, 0u};
  if (n > 1) {
    float mstar = -INFINITY;
    for (int k = 0; k < n; ++k) mstar = fmaxf(mstar, a.part_ml[((int64_t)(i0 + k) * a.H + head) * 2]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < n; ++k) {
      const int64_t slot = (int64_t)(i0 + k) * a.H + head;
      const float wk = exp2f(a.part_ml[slot * 2] - mstar) * a.part_ml[slot * 2 + 1];
      L += wk;
      const u32x2 v = *reinterpret_cast<const u32x2*>((const bf16*)a.part_o + slot * DC + 4 * t);
      acc[0] += wk * bf16_lo(v[0]);
      acc[1] += wk * bf16_hi(v[0]);
      acc[2] += wk * bf16_lo(v[1]);
      acc[3] += wk * bf16_hi(v[1]);
    }
    const float inv = 1.f / L;
    outv[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    outv[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  }
  *reinterpret_cast<u32x2*>(o) = outv;
}

// Work plan: one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void plan_kernel(AttnArgs a, int32_t* plan, int32_t target_items,
                                                    int32_t min_chunk, int32_t max_chunk) {
  __shared__ long long red_tot[32];
  __shared__ int red_max[32];
  __shared__ int scan[1024];
  __shared__ int carry, chunk_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_rows = a.B * a.s_q;
  auto vis = [&](int r) -> int {
    const int b = r / a.s_q, s = r % a.s_q;
    bool ok;
    const int kv = kv_len_of(a, b, ok);
    if (!ok) {
      if (s == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_LEN);
      return 0;
    }
    return kv - a.s_q + s + 1;
  };
  long long tot = 0;
  int mx = 0;
  for (int r = tid; r < n_rows; r += 1024) {
    const int v = vis(r);
    tot += v;
    mx = max(mx, v);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    tot += __shfl_xor(tot, o, 64);
    mx = max(mx, __shfl_xor(mx, o, 64));
  }
  if (lane == 0) {
    red_tot[wv] = tot;
    red_max[wv] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    long long T = 0;
    int M = 0;
    for (int i = 0; i < 16; ++i) {
      T += red_tot[i];
      M = max(M, red_max[i]);
    }
    int chunk = max_chunk;
    if (target_items > 0 && T > 0) {
      // ragged batches get four times as many, smaller, chunks to even out
      const long long tgt = (T * 4 >= 3LL * n_rows * M) ? target_items : 4LL * target_items;
      const long long c = (T + tgt - 1) / tgt;
      chunk = (int)min<long long>(max_chunk, max<long long>(min_chunk, (c + 31) / 32 * 32));
    }
    plan[1] = chunk;
    chunk_s = chunk;
    carry = 0;
  }
  __syncthreads();
  const int chunk = chunk_s;
  for (int base = 0; base < n_rows; base += 1024) {
    const int r = base + tid;
    const int v = r < n_rows ? vis(r) : 0;
    const int c = (v + chunk - 1) / chunk;
    scan[tid] = c;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
      const int x = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += x;
      __syncthreads();
    }
    if (r < n_rows) plan[2 + r] = carry + scan[tid] - c;
    __syncthreads();
    if (tid == 1023) carry += scan[1023];
    __syncthreads();
  }
  if (tid == 0) {
    plan[2 + n_rows] = carry;
    plan[0] = carry;
  }
}

// fp32 reference-shape kernel: one workgroup per (query row, head), any d_c
// <= 1024 and d_rope <= 128, whole visible range in one pass.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  __shared__ float qs[1024 + 128];
  __shared__ float ps[256];
  __shared__ int64_t rowoff[256];
  __shared__ float red[4];
  const int head = blockIdx.x % a.H;
  const int64_t qrow = blockIdx.x / a.H;
  const int b = (int)(qrow / a.s_q), s = (int)(qrow % a.s_q);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int row = a.d_c + a.d_rope;
  float* o = (float*)a.o_lat + (qrow * a.H + head) * a.d_c;
  bool ok;
  const int kv = kv_len_of(a, b, ok);
  if (!ok) {
    if (tid == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_LEN);
    for (int d = tid; d < a.d_c; d += 256) o[d] = 0.f;
    return;
  }
  const int kend = kv - a.s_q + s + 1;
  const float* ql = (const float*)a.q_lat + (qrow * a.H + head) * a.ld_q;
  const float* qr = (const float*)a.q_rope + (qrow * a.H + head) * a.ld_r;
  for (int i = tid; i < a.d_c; i += 256) qs[i] = ql[i];
  for (int i = tid; i < a.d_rope; i += 256) qs[a.d_c + i] = qr[i];
  const float* pool = (const float*)a.pool;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  __syncthreads();
  for (int c0 = 0; c0 < kend; c0 += 256) {
    const int j = c0 + tid;
    float sc = -INFINITY;
    int64_t off = -1;
    if (j < kend) {
      const int pidx = j / a.page_size;
      const int page = pidx < a.max_pages ? bt[pidx] : -1;
      if (page >= 0 && (int64_t)page < a.num_pages) {
        off = ((int64_t)page * a.page_size + j % a.page_size) * row;
        float dot = 0.f;
        for (int x = 0; x < row; ++x) dot += qs[x] * pool[off + x];
        sc = dot * a.scale;
      } else if (a.err_flags) {
        atomicOr(a.err_flags, FLAG_BAD_PAGE);
      }
    }
    rowoff[tid] = off;
    float mw = wave_max(sc);
    if (lane == 0) red[wv] = mw;
    __syncthreads();
    const float mc = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    const float mn = fmaxf(m, mc);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - mn);
    ps[tid] = p;
    float sw = wave_sum(p);
    if (lane == 0) red[wv] = sw;
    __syncthreads();
    const float lc = red[0] + red[1] + red[2] + red[3];
    l = l * alpha + lc;
    m = mn;
    const int nk = min(256, kend - c0);
    for (int r = 0; r < 4; ++r) acc[r] *= alpha;
    for (int jj = 0; jj < nk; ++jj) {
      const int64_t ro = rowoff[jj];
      if (ro < 0) continue;
      const float pj = ps[jj];
      for (int r = 0; r < 4; ++r) {
        const int d = tid + 256 * r;
        if (d < a.d_c) acc[r] += pj * pool[ro + d];
      }
    }
    __syncthreads();
  }
  const float inv = 1.f / l;
  for (int r = 0; r < 4; ++r) {
    const int d = tid + 256 * r;
    if (d < a.d_c) o[d] = acc[r] * inv;
  }
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, hipStream_t st) {
  const int n_hg = (a.H + WG_HEADS - 1) / WG_HEADS;
  const int64_t n = (int64_t)a.max_items * n_hg;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_bf16_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_bf16(const AttnArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.s_q * a.H;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_bf16_kernel, dim3((unsigned)n), dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_plan(const AttnArgs& a, int32_t* plan, int32_t target_items, int32_t min_chunk,
                            int32_t max_chunk, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, st, a, plan, target_items, min_chunk, max_chunk);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.s_q * a.H;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
