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
//
// FP8 cache (the same kernel, FP8 = true): rows are 656 bytes, c^KV as 512
// E4M3 codes, then k^R as 64 bf16, then four fp32 scales 2^e, one per
// 128-value tile of c^KV.  Each tile's codes and k^R (640 bytes a row) move
// by direct-to-LDS loads into one of two staging slots, one tile ahead; the
// workgroup then decodes every value once (v_cvt_scalef32_pk_bf16_fp8: two
// codes per instruction, the power-of-two scale exact) into the bf16 stage
// layout above, so the QK and PV code is the same for both caches.  Three
// bf16 stages then suffice (two read, one written per pass).
#include <math.h>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"

namespace mla {
namespace {

constexpr int DC = 512, DR = 64, ROW = DC + DR;  // cached row: c^KV then k^R
constexpr int TILE = 32;                         // keys per LDS tile
constexpr int RB = ROW * 2;                      // bytes per key row (1152, unpadded)
constexpr int STAGE = TILE * RB;                 // 36864 bytes per tile
// Pass t reads tiles t and t+1 from LDS and issues tile t + DEPTH into the
// stage that held tile t-1: DEPTH - 1 tiles are in flight behind the two in use.
constexpr int DEPTH = 3, NSTAGE = DEPTH + 1;
constexpr int DMA_PER_THREAD = STAGE / 16 / 256; // 9 16-byte loads per thread per tile
constexpr int WG_HEADS = 128;
constexpr int MAX_SPLIT_PAGES = 1536;            // page ids of one split, staged in LDS
constexpr int FLAG_BAD_PAGE = 1, FLAG_BAD_LEN = 4;
// FP8 cache
constexpr int F_RB = 656;                        // bytes per cached row
constexpr int F_SROW = 640;                      // bytes staged per row: codes, then k^R
constexpr int F_SCALE = 640;                     // row offset of the four tile scales
constexpr int F_STAGE = TILE * F_SROW;           // 20480 bytes per staging slot
constexpr int F_NSLOT = 2, F_NSTAGE = 3;
constexpr int F_DMA = F_STAGE / 16 / 256;        // 5 16-byte loads per thread per tile
constexpr int F_SPLIT_PAGES = 512;               // page ids of one split (LDS budget)
static_assert(F_NSTAGE * STAGE + F_NSLOT * F_STAGE + F_SPLIT_PAGES * 4 <= NSTAGE * STAGE + MAX_SPLIT_PAGES * 4,
              "FP8 LDS layout exceeds the bf16 one");
constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_SLACK = 8.0f;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

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

__device__ __forceinline__ float buf_ld4f(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
// two E4M3 codes (bytes 2W, 2W+1 of src) times 2^e (the scale's exponent) as bf16
template <bool W>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t src, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)src, scale, W));
}

template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NST = FP8 ? F_NSTAGE : NSTAGE;             // bf16 tile stages
  constexpr int SPLIT_PAGES = FP8 ? F_SPLIT_PAGES : MAX_SPLIT_PAGES;
  constexpr int NDMA = FP8 ? F_DMA : DMA_PER_THREAD;
  constexpr int RBG = FP8 ? F_RB : RB;                     // bytes per cached row
  __shared__ __attribute__((aligned(16))) unsigned char smem[FP8 ? F_NSTAGE * STAGE + F_NSLOT * F_STAGE
                                                                 : NSTAGE * STAGE];
  __shared__ int split_pages[SPLIT_PAGES];
  __shared__ u32x4 p_xchg[4 * 2 * 64];   // P^T fragments [head block][k step][lane]
  __shared__ float alpha_xchg[4][32];    // per head: rescale factor of the current tile
  __shared__ float lsum_xchg[4][32];     // per head: softmax sum of the chunk
  __shared__ __attribute__((aligned(4))) unsigned char flag_xchg[4];  // head block raised its max this tile

  const int n_hg = (a.H + WG_HEADS - 1) / WG_HEADS;
  const int tid = threadIdx.x;
  // The plan lists this workgroup's item in launch order (the grid is an
  // upper bound on the items; entries past the last item are empty).
  const int bid = (int)blockIdx.x / n_hg, hg = (int)blockIdx.x % n_hg;
  const int4 item = reinterpret_cast<const int4*>(a.plan + plan_info_offset((int64_t)a.B * a.s_q))[bid];
  const int row = __builtin_amdgcn_readfirstlane(item.x);
  const int k0 = __builtin_amdgcn_readfirstlane(item.y), k1 = __builtin_amdgcn_readfirstlane(item.z);
  const int w = __builtin_amdgcn_readfirstlane(item.w) >> 1;         // item index: slot of a partial
  const bool multi = (__builtin_amdgcn_readfirstlane(item.w) & 1) != 0;  // row has several items
  if (k0 >= k1) return;
  const int b = row / a.s_q;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int head0 = hg * WG_HEADS + wave * 32;  // first head of this wave
  const bool wave_on = head0 < a.H;
  const int64_t qrow = row;
  const float scale_log2 = a.scale * LOG2E;

  // ---- the chunk's page ids, staged in LDS (keeping block-table reads off
  // the tile pipeline); waited for before the bulk loads start, so they do
  // not queue behind them
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int pg_first = k0 / a.page_size;
  const int n_pages = (k1 - 1) / a.page_size - pg_first + 1;  // <= SPLIT_PAGES (host plan)
  constexpr int PAGES_PER_THREAD = SPLIT_PAGES / 256;
  int pid[PAGES_PER_THREAD];
#pragma unroll
  for (int k = 0; k < PAGES_PER_THREAD; ++k) {
    const int i = tid + 256 * k, pidx = pg_first + i;
    pid[k] = (i < n_pages && pidx < a.max_pages) ? bt[pidx] : -1;
  }
#pragma unroll
  for (int k = 0; k < PAGES_PER_THREAD; ++k)
    if (tid + 256 * k < n_pages) split_pages[tid + 256 * k] = pid[k];
  __syncthreads();

  // ---- tile loads: wave w's instruction i covers LDS chunks (4i + w)*64 + lane
  // of the stage; LDS chunk P holds key row P / 72, row chunk (P % 72) ^ kswz(row).
  // FP8: of the staging slot, P / 40 and (P % 40) ^ kswz(row) of the row's
  // 40 chunks (32 of codes, 8 of k^R).
  int32_t dma_off[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int P = (4 * i + wave) * 64 + lane;
    constexpr int CPR = FP8 ? F_SROW / 16 : RB / 16;
    const int r = P / CPR, c = (P % CPR) ^ kswz(P / CPR);
    dma_off[i] = r * RBG + c * 16;
  }
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;
  // Issue cursor: the next tile to load sits at key offset cur_off of page
  // slot cur_slot of the chunk (tiles never straddle a page).  Scalar state,
  // advanced by one tile per issue, so no division on the issue path.
  int cur_slot = 0, cur_off = k0 % a.page_size, cur_tile = 0;
  const int ntiles = (k1 - k0 + TILE - 1) / TILE;
  const uint64_t pool_addr = (uint64_t)(uintptr_t)a.pool;
  const uint32_t page_bytes = (uint32_t)a.page_size * RBG;
  const uint32_t num_pages = (uint32_t)min<int64_t>(a.num_pages, 0x7fffffff);
  bool bad_page = false;  // reported once, after the loop
  struct TileDma {
    __amdgpu_buffer_rsrc_t r;
    uint32_t dst;
  };
  // Tiles past the chunk's end are issued too, with an empty resource (their
  // loads write zeros into a free stage): the tile loop then issues and waits
  // for a fixed number of loads per pass, with no branches.
  auto prep_tile = [&](int page_id) {  // resource of the cursor's tile, then advance
    // 32-bit scalar arithmetic only: a negative id fails the unsigned compare
    const uint32_t page = (uint32_t)__builtin_amdgcn_readfirstlane(page_id);
    const bool real = cur_tile < ntiles;
    const bool pok = page < num_pages;
    // rows of the tile are contiguous within one page; rows past k1 (and a
    // bad page) lie outside the resource and load as zeros
    const int kb = k0 + cur_tile * TILE;
    const uint64_t addr = pool_addr + (uint64_t)(pok ? page : 0u) * page_bytes + (uint32_t)cur_off * RBG;
    TileDma d;
    d.r = make_rsrc((const void*)(uintptr_t)addr, (real && pok) ? min(TILE, k1 - kb) * RBG : 0);
    d.dst = FP8 ? smem_addr + F_NSTAGE * STAGE + (cur_tile % F_NSLOT) * F_STAGE + wave * 1024
                : smem_addr + (cur_tile % NSTAGE) * STAGE + wave * 1024;
    cur_tile += 1;
    cur_off += TILE;
    if (cur_off == a.page_size) {
      cur_off = 0;
      cur_slot += 1;
    }
    bad_page |= real && !pok;
    return d;
  };
  // page id at the cursor (a stale id past the chunk: its tile is empty)
  auto cursor_page = [&]() { return split_pages[min(cur_slot, SPLIT_PAGES - 1)]; };
  auto issue_next = [&](int page_id) {
    const TileDma d = prep_tile(page_id);
#pragma unroll
    for (int i = 0; i < NDMA; ++i) dma16(d.r, d.dst + i * 4096, dma_off[i]);
    return d;
  };

  // ---- FP8: decoding of a staged tile into a bf16 stage.  Thread (row
  // r = lane & 31, part p = 2 wave + hi) takes codes 64p .. 64p+63 of row r
  // (all in 128-value tile `wave`, scale `sc`) and k^R chunk p.  Per step:
  // 0..3 read code chunk q, 4 read the k^R chunk (into cvb), 5 + 2q + h decode
  // and store half h of chunk q, 13 store the k^R chunk.
  // Row offsets of this thread's staged and decoded rows (part p's first chunk
  // folded in), and 16 * kswz(row): a chunk index 8a + j (j < 8) swizzles to
  // 8a + (j ^ kswz), so each address is base + (16 j ^ cv_k16).  The XOR is
  // redone at every access (cv_k16 is opaque to the compiler) rather than
  // kept as 14 loop-invariant addresses, which would not fit the registers.
  const int cv_r = lane & 31, cv_p = 2 * wave + hi;
  const int cv_rd = cv_r * F_SROW + 128 * (cv_p >> 1), cv_wr = cv_r * RB + 128 * cv_p;
  const int cv_k16 = 16 * kswz(lane & 31);
  u32x4 cvb = {0u, 0u, 0u, 0u};
  auto cv_step = [&](int step, const unsigned char* F, unsigned char* S, float sc) {
    if constexpr (FP8) {
      int k16 = cv_k16;
      asm volatile("" : "+v"(k16));
      if (step < 4) {  // chunk 4p + step = 8 (p >> 1) + (4 (p & 1) + step)
        cvb = *(const u32x4*)(F + cv_rd + ((16 * (4 * (cv_p & 1) + step)) ^ k16));
      } else if (step < 12) {
        const int q = (step - 4) >> 1, h = (step - 4) & 1;
        u32x4 o;
        o[0] = fp8x2_bf16<false>(cvb[2 * h], sc);
        o[1] = fp8x2_bf16<true>(cvb[2 * h], sc);
        o[2] = fp8x2_bf16<false>(cvb[2 * h + 1], sc);
        o[3] = fp8x2_bf16<true>(cvb[2 * h + 1], sc);
        *(u32x4*)(S + cv_wr + ((16 * (2 * q + h)) ^ k16)) = o;
      } else if (step == 12) {  // k^R chunk 32 + p of the staged row
        cvb = *(const u32x4*)(F + cv_r * F_SROW + 512 + ((16 * cv_p) ^ k16));
      } else {                  // bf16 chunk 64 + p
        *(u32x4*)(S + cv_r * RB + 1024 + ((16 * cv_p) ^ k16)) = cvb;
      }
    }
  };
  auto scale_of = [&](const TileDma& d) { return buf_ld4f(d.r, cv_r * F_RB + F_SCALE + 4 * wave); };
  float scl_cv = 0.f, scl_nx = 0.f;  // scales of the tile decoded next, and of the one after

  // ---- tiles 0 .. DEPTH-2 (possibly empty), then the queries: one burst
  // (bf16: tile DEPTH-1 goes out after the first tile's scores, so the
  // queries, which those scores need whole, are not queued behind it; FP8:
  // tiles 0 and 1 are decoded once they land, tile 2 stays in flight)
  TileDma d0 = issue_next(split_pages[0]);
  if constexpr (FP8) {
    scl_cv = scale_of(d0);
    d0 = issue_next(cursor_page());
    scl_nx = scale_of(d0);
  } else {
#pragma unroll
    for (int p = 1; p < DEPTH - 1; ++p) issue_next(cursor_page());
  }
  // Q^T fragments: B operand of S^T = K Q^T; k step j covers dims 16j .. 16j+15
  // (j < 32: q_lat, j >= 32: q^R).  Heads past H load as zero.
  u32x4 qf[36];
  {
    const int nh = wave_on ? min(32, a.H - head0) : 0;
    const int64_t hrow = qrow * a.H + (wave_on ? head0 : 0);
    const __amdgpu_buffer_rsrc_t ql = make_rsrc((const bf16*)a.q_lat + hrow * a.ld_q, nh * a.ld_q * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc((const bf16*)a.q_rope + hrow * a.ld_r, nh * a.ld_r * 2);
    const int ol = l32 * a.ld_q * 2 + 16 * hi, orr = l32 * a.ld_r * 2 + 16 * hi;
    // issued in the order the first tile's MFMAs use them (sched_barrier keeps
    // the scheduler from reordering), so each MFMA waits only for its own
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      qf[j] = buf_ld16(ql, ol + 32 * j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 32; j < 36; ++j) {
      qf[j] = buf_ld16(qr, orr + 32 * (j - 32));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // bf16: the first tile's scores (before the tile loop) read the query
  // fragments in order, so the compiler's wait for fragment j lets the first
  // MFMAs start while later fragments are still arriving; those waits precede
  // the tile loop, which then never waits for the queries (a wait there would
  // drain the tile loads in flight on every pass).  FP8: the queries are
  // waited for here, with the staged tiles.
  if constexpr (FP8) {
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
                 "v"(qf[7]), "v"(qf[8]), "v"(qf[9]), "v"(qf[10]), "v"(qf[11]));
    asm volatile("" ::"v"(qf[12]), "v"(qf[13]), "v"(qf[14]), "v"(qf[15]), "v"(qf[16]), "v"(qf[17]), "v"(qf[18]),
                 "v"(qf[19]), "v"(qf[20]), "v"(qf[21]), "v"(qf[22]), "v"(qf[23]));
    asm volatile("" ::"v"(qf[24]), "v"(qf[25]), "v"(qf[26]), "v"(qf[27]), "v"(qf[28]), "v"(qf[29]), "v"(qf[30]),
                 "v"(qf[31]), "v"(qf[32]), "v"(qf[33]), "v"(qf[34]), "v"(qf[35]));
  }
  if constexpr (FP8) {
    wait_vmcnt<0>();
    __syncthreads();
    const unsigned char* F0 = smem + F_NSTAGE * STAGE;
#pragma unroll
    for (int t0 = 0; t0 < 2; ++t0) {
      // steps in order: each chunk is read, then decoded in two halves
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cv_step(q, F0 + t0 * F_STAGE, smem + t0 * STAGE, t0 ? scl_nx : scl_cv);
        cv_step(4 + 2 * q, F0 + t0 * F_STAGE, smem + t0 * STAGE, t0 ? scl_nx : scl_cv);
        cv_step(5 + 2 * q, F0 + t0 * F_STAGE, smem + t0 * STAGE, t0 ? scl_nx : scl_cv);
      }
      cv_step(12, F0 + t0 * F_STAGE, smem + t0 * STAGE, 0.f);
      cv_step(13, F0 + t0 * F_STAGE, smem + t0 * STAGE, 0.f);
    }
    __syncthreads();  // staging slot 0 is free again, tiles 0 and 1 are in place
    scl_cv = scale_of(issue_next(cursor_page()));
  }
  // page of the next tile to issue, fetched one tile early to keep the LDS
  // latency off the issue path (bf16: once the prologue's last tile is out)
  int next_page = FP8 ? cursor_page() : 0;

  // Accumulator O^T for this wave's 128 latent dims (4 blocks of 32) and all
  // 128 heads of the workgroup (4 blocks of 32): acc[4 * d + hb].
  f32x16 acc[16];
#pragma unroll
  for (int x = 0; x < 16; ++x)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[x][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // of head head0 + l32 (this wave's head block)

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

  // ---- per-tile pieces ----------------------------------------------------
  // S^T[key][head] for the 32 keys of a tile and this wave's 32 heads, in
  // VGPRs: 36 MFMAs over the 576 dims.  K fragments are read KW steps ahead.
  constexpr int KW = 4;
  u32x4 kf[KW];
  auto qk_begin = [&](const unsigned char* K) {
#pragma unroll
    for (int j = 0; j < KW - 1; ++j) kf[j] = *(const u32x4*)(K + qk_off[j & 3] + 128 * (j >> 2));
  };
  auto qk_step = [&](const unsigned char* K, int j, f32x16& sacc) {
    if (j + KW - 1 < 36) {
      const int jn = j + KW - 1;
      kf[jn % KW] = *(const u32x4*)(K + qk_off[jn & 3] + 128 * (jn >> 2));
    }
    if (j == 0) {
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sacc) : "v"(kf[0]), "v"(qf[0]));
    } else if (j < 35) {
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sacc) : "v"(kf[j % KW]), "v"(qf[j]));
    } else {
      // the trailing wait states let VALU read the MFMA result
      asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
          : "+v"(sacc) : "v"(kf[j % KW]), "v"(qf[j]));
    }
  };
  // Online softmax (log2 domain) of one tile for this wave's heads, cut into
  // slots that run between the next tile's QK MFMAs.  No instruction in a slot
  // depends on another of the same slot (a dependent chain would hold up the
  // in-order issue of the next MFMA).  Lane holds keys kb + 8*(i/4) + 4*hi + i%4
  // of head l32.  The scale is positive, so the max is taken on raw scores and
  // the scale folded into the exponent's FMA.
  constexpr int SM_SLOTS = 27;
  float mx0, mx1, neg_m, alpha = 1.f;
  bool resc = false;  // this tile raised the running max (published with P^T)
  float ex[16];
  u32x4 pf[2];
  auto max3 = [](float x, float y, float z) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
    return r;
  };
  auto sm_slot = [&](int j, f32x16& sc, int kb, bool first) {
    if (j == 1) {
      if (kb + TILE > k1) {  // the chunk's last, partial tile
        const int rem = k1 - kb - 4 * hi;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = (8 * (i >> 2) + (i & 3) < rem) ? sc[i] : -INFINITY;
      }
      mx0 = max3(sc[0], sc[1], sc[2]);
      mx1 = max3(sc[3], sc[4], sc[5]);
    } else if (j == 2) {
      mx0 = max3(mx0, sc[6], sc[7]);
      mx1 = max3(mx1, sc[8], sc[9]);
    } else if (j == 3) {
      mx0 = max3(mx0, sc[10], sc[11]);
      mx1 = max3(mx1, sc[12], sc[13]);
    } else if (j == 4) {
      mx0 = max3(mx0, mx1, sc[14]);
    } else if (j == 5) {
      mx0 = max3(mx0, sc[15], sc[15]);
    } else if (j == 6) {  // the other half of the head's keys sits in lane l ^ 32
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx0), __float_as_uint(mx0), false, false);
      mx0 = __uint_as_float(r[0]);
      mx1 = __uint_as_float(r[1]);
    } else if (j == 7) {
      mx0 = max3(mx0, mx1, mx1) * scale_log2;  // tile max, log2 units
    } else if (j == 8) {
      // running max: raised only when the tile max exceeds it by more than
      // RESCALE_SLACK (p <= 2^8 stays exact); the accumulator rescale is done
      // by every wave after the P^T exchange
      resc = false;
      if (first) {
        m_run = mx0;  // accumulator and sum are still zero
      } else if (__builtin_amdgcn_ballot_w64(mx0 > m_run + RESCALE_SLACK)) {
        resc = true;
        const float mn = fmaxf(m_run, mx0);
        alpha = __builtin_amdgcn_exp2f(m_run - mn);
        l_run *= alpha;
        m_run = mn;
      }
      neg_m = -m_run;
    }
    // P^T fragments: scores 8q .. 8q+7 of this lane are the k slots of step q.
    // Exponents are at most RESCALE_SLACK, so the hardware exp2 needs no range
    // handling (masked keys give exp2(-inf) = 0).  Score i: FMA in slot 9 + i,
    // exp2 in 10 + i; pair k = (2k, 2k+1) is packed and summed in slot 12 + 2k
    // (one transcendental per slot fits under one MFMA; the row sum uses fp32
    // adds, which overlap the MFMAs where a dot2 instruction would not).
    if (j >= 9 && j < 25) ex[j - 9] = __builtin_fmaf(sc[j - 9], scale_log2, neg_m);
    if (j >= 10 && j < 26) ex[j - 10] = __builtin_amdgcn_exp2f(ex[j - 10]);
    if (j >= 12 && j < 27 && (j & 1) == 0) {
      const int k = (j - 12) >> 1;
      pf[k >> 2][k & 3] = pack_bf16x2(ex[2 * k], ex[2 * k + 1]);
      l_run += ex[2 * k] + ex[2 * k + 1];
    }
  };

  // ---- tile loop ------------------------------------------------------------
  // Pass t: QK of tile t+1 (LDS-bound: four waves read every key fragment),
  // then PV of tile t (MFMA-bound) with the softmax of tile t+1 running
  // between its MFMAs; tile t+1's P^T is published after the second barrier.
  // Tiles t and t+1 are read from LDS during pass t, tiles t+2 and t+3 are in
  // flight.
  auto publish = [&]() {  // P^T, rescale flag and factor of this wave's head block
#pragma unroll
    for (int q = 0; q < 2; ++q) p_xchg[(wave * 2 + q) * 64 + lane] = pf[q];
    if (resc) alpha_xchg[wave][l32] = alpha;  // lanes l and l ^ 32 store the same value
    flag_xchg[wave] = resc ? 1 : 0;             // every lane stores the same byte
  };
  f32x16 s_nx;  // scores of the next tile
  // bf16: tile 0 has landed once at most tiles 1 .. DEPTH-2 and the 36 query
  // loads are outstanding (loads complete in order); FP8: everything has
  if constexpr (!FP8) wait_vmcnt<(DEPTH - 2) * DMA_PER_THREAD + 36>();
  __syncthreads();
  {
    const unsigned char* K0 = smem;
    qk_begin(K0);
#pragma unroll
    for (int j = 0; j < 36; ++j) {
      qk_step(K0, j, s_nx);
      __builtin_amdgcn_sched_barrier(0);
    }
    // bf16: tile DEPTH-1, after the last wait for a query fragment (the
    // compiler's waits for them do not count loads issued in asm, so a tile
    // issued earlier would be waited for with them)
    if constexpr (!FP8) {
      issue_next(cursor_page());
      next_page = cursor_page();
    }
#pragma unroll
    for (int j = 0; j < SM_SLOTS; ++j) sm_slot(j, s_nx, k0, true);
    publish();
  }
  // One pass; HAS_NEXT is a compile-time flag so that the interleaved work
  // carries no branches (the last pass is peeled off).
  auto pass = [&](const int t, auto has_next_tag) {
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    // tile t+1 has landed once at most tiles t+2 .. t+DEPTH-1 are outstanding;
    // the barrier makes every thread's loads and tile t's P^T visible (FP8:
    // tile t+2's staged codes, decoded in this pass, and tile t+1's bf16 stage)
    if constexpr (FP8)
      wait_vmcnt<0>();
    else
      wait_vmcnt<(DEPTH - 2) * DMA_PER_THREAD>();
    __syncthreads();
    // tile t+3 (possibly empty) goes to the stage that held tile t-1, read by
    // the previous pass; its loads are spread over this pass's PV MFMAs (all
    // waves issuing at once would queue on the CU's address unit)
    const TileDma nd = prep_tile(next_page);
    next_page = cursor_page();
    // tile t's rescale flags (byte hb for head block hb), read now so the LDS
    // latency is hidden behind the QK phase
    uint32_t flags;
    __builtin_memcpy(&flags, flag_xchg, 4);
    const unsigned char* Kc = smem + (t % NST) * STAGE;
    const int kb_next = k0 + (t + 1) * TILE;
    if constexpr (HAS_NEXT) {
      const unsigned char* Kn = smem + ((t + 1) % NST) * STAGE;
      qk_begin(Kn);
#pragma unroll
      for (int j = 0; j < 36; ++j) {
        qk_step(Kn, j, s_nx);
        // FP8: tile t+3's codes into the staging slot tile t+1 left (decoded
        // in the previous pass), one load after every seventh MFMA
        if constexpr (FP8) {
          if (j == 0) scl_nx = scale_of(nd);
          if (j % 7 == 3 && j / 7 < F_DMA) dma16(nd.r, nd.dst + (j / 7) * 4096, dma_off[j / 7]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- O^T[dim][head] += V^T[dim][key] P^T[key][head] for this wave's 128
    // dims and all 128 heads: per k step q, 4 dim blocks x 4 head blocks.
    constexpr int VW = 3;  // V fragments in flight
    auto load_v = [&](int m) {  // fragment m: k step m >> 2, dim block 4 * wave + (m & 3)
      const int q = m >> 2, d = m & 3;
      const unsigned char* Kd = Kc + 256 * wave + 128 * (d >> 1);
      const u32x2 lo = lds_tr16(Kd + pv_off[q][0][d & 1]);
      const u32x2 hv = lds_tr16(Kd + pv_off[q][1][d & 1]);
      return u32x4{lo[0], lo[1], hv[0], hv[1]};
    };
    u32x4 pb[4];  // P^T fragments of the current k step; step 1 reloads them in place
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) pb[hb] = p_xchg[hb * 2 * 64 + lane];
    u32x4 vf[VW];
#pragma unroll
    for (int i = 0; i < VW - 1; ++i) vf[i] = load_v(i);

    // ---- rescale the accumulator columns of head blocks whose max was raised
    flags = __builtin_amdgcn_readfirstlane(flags);
    if (flags) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        if ((flags >> (8 * hb)) & 1) {
          const float al = alpha_xchg[hb][l32];
          asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
          for (int d = 0; d < 4; ++d) scale_acc_tuple(acc[4 * d + hb], al);
          asm volatile("s_nop 4" ::: "memory");
        }
      }
    }

#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int m = 4 * q + d;
        if (m + VW - 1 < 8) vf[(m + VW - 1) % VW] = load_v(m + VW - 1);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          if (m == 0 && hb == 0) {
            asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                : "+a"(acc[4 * d + hb]) : "v"(vf[m % VW]), "v"(pb[hb]));
          } else {
            asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                : "+a"(acc[4 * d + hb]) : "v"(vf[m % VW]), "v"(pb[hb]));
          }
          // after its last use in step 0, the fragment is reloaded for step 1
          if (q == 0 && d == 3) pb[hb] = p_xchg[(hb * 2 + 1) * 64 + lane];
          const int mi = 4 * m + hb;
          // the next tile's softmax, one slot per MFMA
          if constexpr (HAS_NEXT) {
            if (mi < SM_SLOTS) sm_slot(mi, s_nx, kb_next, false);
          }
          if constexpr (FP8) {
            // decode tile t+2 (staged in the previous pass) into the stage
            // tile t-1 left: chunk c read after MFMA 7c, its halves after
            // 7c+3 and 7c+5; the k^R chunk read after 28, stored after 30
            unsigned char* S = smem + ((t + 2) % F_NSTAGE) * STAGE;
            const unsigned char* F = smem + F_NSTAGE * STAGE + (t % F_NSLOT) * F_STAGE;
            if (mi < 28 && mi % 7 == 0) cv_step(mi / 7, F, S, scl_cv);
            if (mi < 28 && mi % 7 == 3) cv_step(4 + 2 * (mi / 7), F, S, scl_cv);
            if (mi < 28 && mi % 7 == 5) cv_step(5 + 2 * (mi / 7), F, S, scl_cv);
            if (mi == 28) cv_step(12, F, S, scl_cv);
            if (mi == 30) cv_step(13, F, S, scl_cv);
          } else {
            // one of tile t+3's loads after every third MFMA
            if (mi % 3 == 1 && mi / 3 < DMA_PER_THREAD) dma16(nd.r, nd.dst + (mi / 3) * 4096, dma_off[mi / 3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    if constexpr (FP8) scl_cv = scl_nx;
    // every wave is done with tile t's P^T and rescale slots
    __syncthreads();
    if constexpr (HAS_NEXT) publish();
  };
  for (int t = 0; t + 1 < ntiles; ++t) pass(t, BoolTag<true>{});
  pass(ntiles - 1, BoolTag<false>{});
  wait_vmcnt<0>();  // the empty tiles' loads still write LDS: drain them
  // wait states before VALU reads of accumulators last written by an MFMA
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0]), "+a"(acc[1]), "+a"(acc[2]), "+a"(acc[3]), "+a"(acc[4]), "+a"(acc[5]),
                 "+a"(acc[6]), "+a"(acc[7]), "+a"(acc[8]), "+a"(acc[9]), "+a"(acc[10]), "+a"(acc[11]),
                 "+a"(acc[12]), "+a"(acc[13]), "+a"(acc[14]), "+a"(acc[15]));

  if (bad_page && tid == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_PAGE);
  // Each head block's owner publishes its softmax sums.
  const float l_tot = pair_sum32(l_run);
  if (hi == 0) lsum_xchg[wave][l32] = l_tot;
  __syncthreads();
  // normalised by this chunk's sum: the final output when the row is one
  // chunk, else a partial the merge combines with weights 2^(m - m*) * l.
  // Lane (l32, hi), tuple (d, hb), register 4g + e holds dim
  // 128 wave + 32 d + 8 g + 4 hi + e of head 128 hg + 32 hb + l32.  Lanes l
  // and l + 32 trade halves (v_permlane32_swap: lanes 32..63 of the first
  // operand with lanes 0..31 of the second) so each stores 8 whole dims.
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const int head = hg * WG_HEADS + 32 * hb + l32;
    if (head >= a.H) break;
    const float inv = 1.f / lsum_xchg[hb][l32];
    bf16* o = (!multi ? (bf16*)a.o_lat + (qrow * a.H + head) * DC
                      : (bf16*)a.part_o + ((int64_t)w * a.H + head) * DC) + 128 * wave;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {  // dim groups g0 = 2 gp, g1 = 2 gp + 1
        const f32x16& t = acc[4 * d + hb];
        uint32_t own[2][2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g = 2 * gp + k;
          own[k][0] = pack_bf16x2(t[4 * g] * inv, t[4 * g + 1] * inv);
          own[k][1] = pack_bf16x2(t[4 * g + 2] * inv, t[4 * g + 3] * inv);
        }
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(own[0][e], own[1][e], false, false);
          v[e] = r[0];
          v[2 + e] = r[1];
        }
        // lane hi = 0 now holds dims 8 g0 .. 8 g0 + 7, lane hi = 1 dims 8 g1 .. 8 g1 + 7
        *reinterpret_cast<u32x4*>(o + 32 * d + 8 * (2 * gp + hi)) = v;
      }
  }
  if (multi && hi == 0 && head0 + l32 < a.H) {
    const int64_t slot = (int64_t)w * a.H + head0 + l32;
    a.part_ml[slot * 2] = m_run;
    a.part_ml[slot * 2 + 1] = l_tot;
  }
}

// Merge of split partials o_k = acc_k / l_k (m_k in the log2 domain):
//   o_lat = sum_k 2^(m_k - m*) l_k o_k / sum_k 2^(m_k - m*) l_k,  m* = max_k m_k.
// Rows cut into a single chunk were written by the attention kernel; rows
// with no chunk (invalid length) are written as zero.  One workgroup per
// (row, 4 heads): 64 threads per head, 8 dims (16 bytes) per thread; the
// loads of up to MERGE_BATCH splits are issued together.
constexpr int MERGE_BATCH = 8;
__global__ __launch_bounds__(256) void merge_bf16_kernel(AttnArgs a) {
  const int hq = a.H / 4;
  const int64_t row = blockIdx.x / hq;
  const int head = (int)(blockIdx.x % hq) * 4 + (threadIdx.x >> 6);
  const int t = threadIdx.x & 63;
  const int32_t* row_off = a.plan + 2;
  const int i0 = row_off[row], n = row_off[row + 1] - i0;
  if (n == 1) return;
  u32x4 outv = {0u, 0u, 0u, 0u};
  if (n > 1) {
    // all (m, l) pairs and partial vectors of a batch are loaded before use
    float mstar = -INFINITY, L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n; k0 += MERGE_BATCH) {
      u32x4 v[MERGE_BATCH];
      float mk[MERGE_BATCH], lk[MERGE_BATCH];
#pragma unroll
      for (int k = 0; k < MERGE_BATCH; ++k) {
        if (k0 + k < n) {
          const int64_t slot = (int64_t)(i0 + k0 + k) * a.H + head;
          const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + slot * 2);
          mk[k] = ml.x;
          lk[k] = ml.y;
          v[k] = *reinterpret_cast<const u32x4*>((const bf16*)a.part_o + slot * DC + 8 * t);
        }
      }
      // running rescale across batches (one batch for up to MERGE_BATCH splits)
      float mb = mstar;
#pragma unroll
      for (int k = 0; k < MERGE_BATCH; ++k)
        if (k0 + k < n) mb = fmaxf(mb, mk[k]);
      const float alpha = exp2f(mstar - mb);
      L *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
      mstar = mb;
#pragma unroll
      for (int k = 0; k < MERGE_BATCH; ++k) {
        if (k0 + k < n) {
          const float wk = exp2f(mk[k] - mstar) * lk[k];
          L += wk;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            acc[2 * d] += wk * bf16_lo(v[k][d]);
            acc[2 * d + 1] += wk * bf16_hi(v[k][d]);
          }
        }
      }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int d = 0; d < 4; ++d) outv[d] = pack_bf16x2(acc[2 * d] * inv, acc[2 * d + 1] * inv);
  }
  *reinterpret_cast<u32x4*>((bf16*)a.o_lat + (row * a.H + head) * DC + 8 * t) = outv;
}

// Merge of the split partials fused with o = W_i^UV o_lat (a6 and a7 in one
// pass, for up to a few hundred query rows).  Workgroup = (head, 32 query
// rows), 4 waves.  Phase 1: the 32 rows' o_lat (one chunk: the attention
// kernel's o_lat; several: the merge above, in registers) go to LDS as bf16.
// Phase 2: out[r, head, n] = sum_k o_lat[r, k] W^UV[head*128 + n, k] on the
// MFMA, wave w taking n = 32w .. 32w+31; W^UV's rows are loaded straight into
// B-operand registers at the start, so they arrive during phase 1.
constexpr int MW_ROWS = 32, MW_RS = DC * 2 + 16;  // rows per workgroup; LDS row stride (bytes)
constexpr int MW_BATCH = 4;                       // split partials per row loaded together
__global__ __launch_bounds__(256) void merge_wuv_bf16_kernel(AttnArgs a, const bf16* __restrict__ w_uv,
                                                             bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char ot[MW_ROWS * MW_RS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int H = a.H, head = (int)(blockIdx.x % H);
  const int r0 = (int)(blockIdx.x / H) * MW_ROWS;
  const int n_rows = a.B * a.s_q;
  // B operand of step s: W^UV row head*128 + 32 wave + l32, columns 16 s + 8 hi .. + 7
  const bf16* wrow = w_uv + ((int64_t)head * 128 + 32 * wave + l32) * DC + 8 * hi;
  u32x4 bw[DC / 16];
#pragma unroll
  for (int s = 0; s < DC / 16; ++s) bw[s] = ld16(wrow + 16 * s);

  // phase 1: thread handles 16-byte chunk `lane` of rows wave + 4 i, i < 8.
  // The loads of all eight rows (up to MW_BATCH partials each) are issued
  // before any is used; a row with more partials finishes in a loop.
  constexpr int NR = MW_ROWS / 4;
  const int32_t* row_off = a.plan + 2;
  int i0[NR], n[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {  // (unguarded: a row past the batch reads the last row's offsets)
    const int r = r0 + wave + 4 * i, rc = min(r, max(n_rows - 1, 0));
    const int b0 = row_off[rc], b1 = row_off[rc + 1];
    i0[i] = r < n_rows ? b0 : 0;
    n[i] = r < n_rows ? b1 - b0 : 0;
  }
  u32x4 v[NR][MW_BATCH];
  float mk[NR][MW_BATCH], lk[NR][MW_BATCH];
  // The loads are unguarded (a slot past a row's last reads the last one, a
  // row with one chunk reads its o_lat row, a row past the batch the last
  // row's) and the unused values are dropped by selects: guarded loads each
  // waited for the one before.
  const int last_row = max(n_rows - 1, 0);
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + wave + 4 * i;
    const bool one = n[i] == 1;  // one chunk: the attention kernel wrote o_lat itself
    const int last = max(n[i] - 1, 0);
    const bf16* orow = (const bf16*)a.o_lat + ((int64_t)min(r, last_row) * H + head) * DC + 8 * lane;
#pragma unroll
    for (int k = 0; k < MW_BATCH; ++k) {
      const int64_t slot = (int64_t)(i0[i] + min(k, last)) * H + head;
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + slot * 2);
      const u32x4 x = ld16(one ? orow : (const bf16*)a.part_o + slot * DC + 8 * lane);
      const bool valid = one ? k == 0 : k < n[i];
      v[i][k] = valid ? x : u32x4{0u, 0u, 0u, 0u};
      mk[i][k] = valid ? (one ? 0.f : ml.x) : -INFINITY;
      lk[i][k] = valid ? (one ? 1.f : ml.y) : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float mstar = -INFINITY, L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // o = sum_k 2^(m_k - m*) l_k o_k / sum_k 2^(m_k - m*) l_k over batches of partials
    auto add_batch = [&](const u32x4 (&vb)[MW_BATCH], const float (&mb_)[MW_BATCH], const float (&lb)[MW_BATCH]) {
      float mb = mstar;
#pragma unroll
      for (int k = 0; k < MW_BATCH; ++k) mb = fmaxf(mb, mb_[k]);
      const float alpha = mb == -INFINITY ? 1.f : exp2f(mstar - mb);  // (no branch on loaded values)
      L *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
      mstar = mb;
#pragma unroll
      for (int k = 0; k < MW_BATCH; ++k) {
        const float wk = lb[k] > 0.f ? exp2f(mb_[k] - mstar) * lb[k] : 0.f;
        L += wk;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] += wk * bf16_lo(vb[k][d]);
          acc[2 * d + 1] += wk * bf16_hi(vb[k][d]);
        }
      }
    };
    add_batch(v[i], mk[i], lk[i]);
    for (int k0 = MW_BATCH; k0 < n[i]; k0 += MW_BATCH) {  // rows with more partials
      u32x4 vb[MW_BATCH];
      float mb_[MW_BATCH], lb[MW_BATCH];
#pragma unroll
      for (int k = 0; k < MW_BATCH; ++k) {
        const int64_t slot = (int64_t)(i0[i] + min(k0 + k, n[i] - 1)) * H + head;
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + slot * 2);
        const u32x4 x = ld16((const bf16*)a.part_o + slot * DC + 8 * lane);
        const bool valid = k0 + k < n[i];
        mb_[k] = valid ? ml.x : -INFINITY;
        lb[k] = valid ? ml.y : 0.f;
        vb[k] = valid ? x : u32x4{0u, 0u, 0u, 0u};
      }
      add_batch(vb, mb_, lb);
    }
    u32x4 res = {0u, 0u, 0u, 0u};
    if (L > 0.f) {
      const float inv = 1.f / L;
#pragma unroll
      for (int d = 0; d < 4; ++d) res[d] = pack_bf16x2(acc[2 * d] * inv, acc[2 * d + 1] * inv);
    }
    *reinterpret_cast<u32x4*>(ot + (wave + 4 * i) * MW_RS + 16 * lane) = res;
  }
  __syncthreads();

  // phase 2: D[row][n] over the 32 rows and this wave's 32 columns
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < DC / 16; ++s)
    acc = mfma32(*reinterpret_cast<const u32x4*>(ot + l32 * MW_RS + (2 * s + hi) * 16), bw[s], acc);
  // lane (l32, hi), register 4 g + e: row 8 g + 4 hi + e, column 32 wave + l32
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = r0 + 8 * (i >> 2) + 4 * hi + (i & 3);
    if (r < n_rows) out[((int64_t)r * H + head) * 128 + 32 * wave + l32] = (bf16)acc[i];
  }
}

// The same merge and W^UV for a few query rows with many splits each (long
// contexts): one workgroup per (row, head), so the grid has rows x H
// workgroups instead of H, and the row's partials are shared out over the
// four waves (wave w takes splits w, w + 4, ...), each keeping four loads in
// flight; the waves' (m*, L, acc) are combined through LDS.  o_lat goes to
// row 0 of the 32-row MFMA operand and only output row 0 is stored.
// Workgroup ids run head-fastest, so the workgroups of one head (sharing
// W_i^UV) are on one XCD.
constexpr int MR_BATCH = 4;  // partials per wave loaded together
__global__ __launch_bounds__(256) void merge_wuv_row_bf16_kernel(AttnArgs a, const bf16* __restrict__ w_uv,
                                                                 bf16* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) unsigned char ot[MW_ROWS * MW_RS];
  __shared__ float cm[4], cl[4];
  __shared__ __attribute__((aligned(16))) float cacc[4][DC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int H = a.H, head = (int)(blockIdx.x % H), r = (int)(blockIdx.x / H);
  // B operand of step s: W^UV row head*128 + 32 wave + l32, columns 16 s + 8 hi .. + 7
  const bf16* wrow = w_uv + ((int64_t)head * 128 + 32 * wave + l32) * DC + 8 * hi;
  u32x4 bw[DC / 16];
#pragma unroll
  for (int s = 0; s < DC / 16; ++s) bw[s] = ld16(wrow + 16 * s);

  const int32_t* row_off = a.plan + 2;
  const int i0 = row_off[r], n = row_off[r + 1] - i0;
  float mstar = -INFINITY, L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n == 1) {  // one chunk: the attention kernel wrote o_lat itself
    if (wave == 0) {
      const u32x4 x = ld16((const bf16*)a.o_lat + ((int64_t)r * H + head) * DC + 8 * lane);
      mstar = 0.f;
      L = 1.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] = bf16_lo(x[d]);
        acc[2 * d + 1] = bf16_hi(x[d]);
      }
    }
  } else {
    for (int k0 = wave; k0 < n; k0 += 4 * MR_BATCH) {
      u32x4 vb[MR_BATCH];
      float mb_[MR_BATCH], lb[MR_BATCH];
      // unguarded loads (a split past the row's last reads the last one and
      // is dropped by the selects), so all of a batch's loads are in flight
      // together: guarded ones each waited for the one before
#pragma unroll
      for (int k = 0; k < MR_BATCH; ++k) {
        const int kk = k0 + 4 * k;
        const int64_t slot = (int64_t)(i0 + min(kk, n - 1)) * H + head;
        const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + slot * 2);
        const u32x4 x = ld16((const bf16*)a.part_o + slot * DC + 8 * lane);
        const bool valid = kk < n;
        mb_[k] = valid ? ml.x : -INFINITY;
        lb[k] = valid ? ml.y : 0.f;
        vb[k] = valid ? x : u32x4{0u, 0u, 0u, 0u};
      }
      float mb = mstar;
#pragma unroll
      for (int k = 0; k < MR_BATCH; ++k) mb = fmaxf(mb, mb_[k]);
      // (no branch on the loaded values: it would hold up the batch's loads)
      const float alpha = mb == -INFINITY ? 1.f : exp2f(mstar - mb);
      L *= alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[d] *= alpha;
      mstar = mb;
#pragma unroll
      for (int k = 0; k < MR_BATCH; ++k) {
        const float wk = lb[k] > 0.f ? exp2f(mb_[k] - mstar) * lb[k] : 0.f;
        L += wk;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] += wk * bf16_lo(vb[k][d]);
          acc[2 * d + 1] += wk * bf16_hi(vb[k][d]);
        }
      }
    }
  }
  // combine the four waves: o = sum_w 2^(m_w - M) acc_w / sum_w 2^(m_w - M) L_w
  if (lane == 0) {
    cm[wave] = mstar;
    cl[wave] = L;
  }
  *reinterpret_cast<f32x4*>(&cacc[wave][8 * lane]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<f32x4*>(&cacc[wave][8 * lane + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  __syncthreads();
  if (wave == 0) {
    const float M = fmaxf(fmaxf(cm[0], cm[1]), fmaxf(cm[2], cm[3]));
    float Lt = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = cl[w] > 0.f ? exp2f(cm[w] - M) : 0.f;
      Lt += sc * cl[w];
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&cacc[w][8 * lane]);
      const f32x4 hv = *reinterpret_cast<const f32x4*>(&cacc[w][8 * lane + 4]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        o[d] += sc * lo[d];
        o[4 + d] += sc * hv[d];
      }
    }
    u32x4 res = {0u, 0u, 0u, 0u};
    if (Lt > 0.f) {
      const float inv = 1.f / Lt;
#pragma unroll
      for (int d = 0; d < 4; ++d) res[d] = pack_bf16x2(o[2 * d] * inv, o[2 * d + 1] * inv);
    }
    *reinterpret_cast<u32x4*>(ot + 16 * lane) = res;  // row 0 of the A operand
  }
  __syncthreads();
  // out[r, head, n] = sum_k o_lat[r, k] W^UV[head*128 + n, k]: rows 1..31 of the
  // operand are not read into any stored value (each output row depends on its
  // own operand row only)
  f32x16 accm;
#pragma unroll
  for (int i = 0; i < 16; ++i) accm[i] = 0.f;
#pragma unroll
  for (int s = 0; s < DC / 16; ++s)
    accm = mfma32(*reinterpret_cast<const u32x4*>(ot + l32 * MW_RS + (2 * s + hi) * 16), bw[s], accm);
  // lane (l32, hi = 0), register 0: row 0, column 32 wave + l32
  if (hi == 0) out[((int64_t)r * H + head) * 128 + 32 * wave + l32] = (bf16)accm[0];
}

// Work plan: one workgroup of 256 threads (wave-level scans, three barriers
// per 256 rows).
__global__ __launch_bounds__(256) void plan_kernel(AttnArgs a, int32_t* plan, int32_t target_items,
                                                   int32_t min_chunk, int32_t max_chunk) {
  plan_body(a, plan, target_items, min_chunk, max_chunk);
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
  if (a.fp8)
    hipLaunchKernelGGL(attn_bf16_kernel<true>, dim3((unsigned)n), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_bf16_kernel<false>, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_bf16(const AttnArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.s_q * (a.H / 4);  // H is a multiple of 32 on this path
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_bf16_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_merge_wuv_bf16(const AttnArgs& a, const void* w_uv, void* out, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * a.s_q;
  if (rows <= 0) return hipSuccess;
  if (rows <= MW_ROWS) {  // a few rows: one workgroup per (row, head)
    hipLaunchKernelGGL(merge_wuv_row_bf16_kernel, dim3((unsigned)(rows * a.H)), dim3(256), 0, st, a,
                       (const bf16*)w_uv, (bf16*)out);
    return hipGetLastError();
  }
  const int64_t n = (int64_t)a.H * ((rows + MW_ROWS - 1) / MW_ROWS);
  hipLaunchKernelGGL(merge_wuv_bf16_kernel, dim3((unsigned)n), dim3(256), 0, st, a, (const bf16*)w_uv, (bf16*)out);
  return hipGetLastError();
}

hipError_t launch_attn_plan(const AttnArgs& a, int32_t* plan, int32_t target_items, int32_t min_chunk,
                            int32_t max_chunk, hipStream_t st) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a, plan, target_items, min_chunk, max_chunk);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.B * a.s_q * a.H;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_f32_kernel, dim3((unsigned)n), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
