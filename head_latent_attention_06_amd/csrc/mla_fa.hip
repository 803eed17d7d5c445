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

#include <algorithm>
#include <utility>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int FA_DH = 128, FA_DR = 64;        // d_h (q^C, k^C, v^C) and d_h^R
constexpr int FA_KT = 64;                     // keys per tile
constexpr int FA_QW = 64, FA_QG = 4 * FA_QW;  // queries per wave / per workgroup
// LDS: a ring of FA_NK key stages (k^C rows of 256 B, then k^R rows of
// 128 B, 64 keys) and a ring of FA_NV value stages (v^C rows of 256 B).  While
// tile t's softmax runs, tile t+1's keys and tile t-1's values are read and
// tiles t+2, t+3 are in flight, so key rows live 3 tile steps and value rows 5.
constexpr int FA_KR = FA_KT * 256, FA_KSTAGE = FA_KR + FA_KT * 128;  // 24576
constexpr int FA_VSTAGE = FA_KT * 256;                               // 16384
constexpr int FA_NK = 3, FA_NV = 5;
constexpr int FA_VBASE = FA_NK * FA_KSTAGE;
constexpr int FA_LDS = FA_VBASE + FA_NV * FA_VSTAGE;  // 155648 bytes
constexpr int FA_DMA = 10;                    // 16-byte loads per thread per tile
constexpr float FA_LOG2E = 1.4426950408889634f;
constexpr float FA_SLACK = 8.0f;

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};
// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}),
// each a separate instantiation, so every index is a compile-time constant
template <typename F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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
// LDS reads at a byte address within the workgroup's LDS
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short fa_s16x4;
__device__ __forceinline__ u32x2 fa_tr16(uint32_t addr) {
  const fa_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) fa_s16x4*)addr);
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 fa_lds16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)addr;
}
template <typename T>
__device__ __forceinline__ const T* fa_uniform(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// Causal mask of one 32x32 S^T tuple in place: register i of the lane holds
// key row 8 (i/4) + i%4 (plus the lane's offset folded into thr); rows past
// thr become -inf.  In asm so the tuple keeps its registers.
__device__ __forceinline__ void fa_causal_mask(f32x16& s, int thr) {
#define FA_MASK1(i, c) "v_cmp_gt_i32 vcc, " #c ", %16\n\tv_cndmask_b32 %" #i ", %" #i ", %17, vcc\n\t"
  asm volatile(FA_MASK1(0, 0) FA_MASK1(1, 1) FA_MASK1(2, 2) FA_MASK1(3, 3) FA_MASK1(4, 8) FA_MASK1(5, 9)
               FA_MASK1(6, 10) FA_MASK1(7, 11) FA_MASK1(8, 16) FA_MASK1(9, 17) FA_MASK1(10, 18) FA_MASK1(11, 19)
               FA_MASK1(12, 24) FA_MASK1(13, 25) FA_MASK1(14, 26) FA_MASK1(15, 27)
               : "+v"(s[0]), "+v"(s[1]), "+v"(s[2]), "+v"(s[3]), "+v"(s[4]), "+v"(s[5]), "+v"(s[6]), "+v"(s[7]),
                 "+v"(s[8]), "+v"(s[9]), "+v"(s[10]), "+v"(s[11]), "+v"(s[12]), "+v"(s[13]), "+v"(s[14]),
                 "+v"(s[15])
               : "v"(thr), "v"(-INFINITY)
               : "vcc");
#undef FA_MASK1
}
// The MFMA order of a tile step: per key step of the value product, units
// "QPQPQPQPQOQ" (Q: a score fragment, P: value block d = 0..3, O: row sum),
// 44 units in all (24 Q, 16 P, 4 O).
constexpr char fa_unit_kind(int u) { return "QPQPQPQPQOQ"[u % 11]; }
constexpr int fa_unit_q(int u) {  // score fragment of unit u (0..23)
  int n = 0;
  for (int v = 0; v < u; ++v) n += fa_unit_kind(v) == 'Q';
  return n;
}
constexpr int fa_unit_load(int u) {  // position of unit u's fragment in load order (0..39)
  int n = 0;
  for (int v = 0; v < u; ++v) n += fa_unit_kind(v) != 'O';
  return n;
}
constexpr int fa_load_unit(int g) {  // unit whose fragment is load g
  for (int u = 0; u < 44; ++u)
    if (fa_unit_kind(u) != 'O' && fa_unit_load(u) == g) return u;
  return -1;
}
// max of three floats (v_max3_f32; the inputs are never signalling NaNs)
__device__ __forceinline__ float fa_max3(float x, float y, float z) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
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

// One work item: 256 queries of one head of one sequence, its key tiles
// taken in ascending order, or in descending order when desc is set (the
// online softmax does not depend on the order; the schedule below uses it to
// keep workgroups on the same keys).  The caller separates consecutive items
// by a barrier.
__device__ __forceinline__ void fa_item(const FaArgs& a, const int work, const bool desc) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[FA_LDS];
  // opaque, so the per-lane values below are computed per item rather than
  // hoisted out of the caller's item loop (where they would stay live)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  // work id -> (sequence, head, query group): the query groups of one head are
  // consecutive ids, longest first
  const int H = a.H;
  const int n_qg = (a.L + FA_QG - 1) / FA_QG;
  const int q0 = (n_qg - 1 - work % n_qg) * FA_QG;
  const int head = (work / n_qg) % H, b = work / n_qg / H;
  // keys [0, start_pos + last query of the workgroup]
  const int kv_hi = a.start_pos + min(q0 + FA_QG, a.L);
  const int ntiles = (kv_hi + FA_KT - 1) / FA_KT;
  // Tile steps run in pairs (the two score and P^T buffers swap roles): the
  // workgroup passes nt_all steps, ntiles rounded up to even.  Step t takes
  // key tile t, or nt_all - 1 - t in descending order; a tile past kv_hi
  // (the rounding, and steps past nt_all whose loads are issued by the
  // pipeline) loads as zeros and is masked by causality.
  const int nt_all = (ntiles + 1) & ~1;
  auto key_tile = [&](int t) { return desc ? nt_all - 1 - t : t; };
  const float scale_log2 = a.scale * FA_LOG2E;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  // ---- tile loads.  k^C / v^C rows of this head: H*128 bf16 apart; k^R rows:
  // ld_kr bf16 apart.  LDS chunk swizzles (16-byte chunk c of row r):
  //   k^C: c ^ (r & 15)        k^R: c ^ ((r >> 1) & 7)        v^C: c ^ 4 (r & 3)
  // make the QK fragment reads and the transposing V reads conflict-free.
  const int64_t krow_bytes = (int64_t)H * FA_DH * 2;
  // Instruction i of wave w moves rows 4 (4i + w) .. +3 (k^C, v^C: 16 chunks
  // per row) or 8 (4i + w) .. +7 (k^R: 8 chunks); the swizzle of those rows
  // depends on the lane only.  Each load's per-lane offset (its rows and the
  // lane's swizzled chunk) is fixed for the whole kernel, so a tile needs one
  // buffer resource per source, bounded by its valid rows (rows past the end
  // are outside it and load as zero), and a load costs an M0 write and the
  // load itself.
  const int ldkr2 = a.ld_kr * 2;
  const int32_t dkc = (int32_t)((lane >> 4) * krow_bytes) + 16 * ((lane & 15) ^ (4 * wave + (lane >> 4)));
  const int32_t dvc = (int32_t)((lane >> 4) * krow_bytes) + 16 * ((lane & 15) ^ (4 * (lane >> 4)));
  const int32_t dkr = (lane >> 3) * ldkr2 + 16 * ((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7));
  int32_t voff[FA_DMA];  // n < 8: k^C (n even) / v^C (n odd) rows 4 (4 (n/2) + w) ..; n >= 8: k^R rows 8 (4 (n-8) + w) ..
#pragma unroll
  for (int n = 0; n < FA_DMA; ++n)
    voff[n] = n < 8 ? (int32_t)(4 * (4 * (n >> 1) + wave) * krow_bytes) + ((n & 1) ? dvc : dkc)
                    : 8 * (4 * (n - 8) + wave) * ldkr2 + dkr;
  const int64_t key_base = (int64_t)b * a.kv_end;
  struct TileSrc {
    __amdgpu_buffer_rsrc_t rk, rv, rr;
    uint32_t ks, vs;
  };
  auto tile_src = [&](int t) {
    const int kt = key_tile(t);
    const int kb0 = max(kt, 0) * FA_KT;
    const int rows = kt < 0 ? 0 : max(0, min(FA_KT, kv_hi - kb0));
    TileSrc ts;
    const int32_t nb_kv = __builtin_amdgcn_readfirstlane(rows > 0 ? (int32_t)((rows - 1) * krow_bytes + FA_DH * 2) : 0);
    const int32_t nb_r = __builtin_amdgcn_readfirstlane(rows > 0 ? (rows - 1) * ldkr2 + FA_DR * 2 : 0);
    ts.rk = fa_rsrc(fa_uniform((const unsigned char*)a.kc + ((key_base + kb0) * H * FA_DH + head * FA_DH) * 2), nb_kv);
    ts.rv = fa_rsrc(fa_uniform((const unsigned char*)a.vc + ((key_base + kb0) * H * FA_DH + head * FA_DH) * 2), nb_kv);
    ts.rr = fa_rsrc(fa_uniform((const unsigned char*)a.kr + (key_base + kb0) * ldkr2), nb_r);
    ts.ks = __builtin_amdgcn_readfirstlane(smem_addr + (t % FA_NK) * FA_KSTAGE);
    ts.vs = __builtin_amdgcn_readfirstlane(smem_addr + FA_VBASE + (t % FA_NV) * FA_VSTAGE);
    return ts;
  };
  auto dma_one = [&](const TileSrc& ts, int n) {
    if (n < 8) {
      const int i = n >> 1;
      if (n & 1)
        fa_dma16(ts.rv, ts.vs + (4 * i + wave) * 1024, voff[n]);
      else
        fa_dma16(ts.rk, ts.ks + (4 * i + wave) * 1024, voff[n]);
    } else {
      fa_dma16(ts.rr, ts.ks + FA_KR + (4 * (n - 8) + wave) * 1024, voff[n]);
    }
  };
  auto issue_tile = [&](int t) {
    const TileSrc ts = tile_src(t);
#pragma unroll
    for (int n = 0; n < FA_DMA; ++n) dma_one(ts, n);
  };
  issue_tile(0);
  issue_tile(1);
  issue_tile(2);

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

  // Per-lane LDS read addresses.  QK A operand: key row 32 kb + l32, chunk
  // 2s + hi (k^C) or 2s' + hi (k^R); V^T A operand via transposing reads: key
  // step ks, read r: row 16 ks + 8 r + 4 hi + jl/4, dim block d: chunk
  // 4 d + 2 g1 + (jl&3)/2, half jl & 1.  With the swizzles above, the address
  // of fragment s (or d) is a per-lane base XOR 32 s (64 d): the stage bases
  // and the smem base have no bits where s and d land.
  const int g1 = (lane >> 4) & 1, jl = lane & 15, rl = 4 * hi + (jl >> 2);
  const uint32_t kx = l32 * 256 + 16 * (hi ^ (l32 & 1)) + 32 * ((l32 & 15) >> 1);
  const uint32_t rx = FA_KR + l32 * 128 + 16 * (hi ^ ((l32 >> 1) & 1)) + 32 * (((l32 >> 1) & 7) >> 1);
  const uint32_t vx = rl * 256 + 64 * (rl & 3) + 32 * g1 + 16 * ((jl & 3) >> 1) + 8 * (jl & 1);

  f32x16 acc[4][2];  // O^T [dim block][query block], AGPRs
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[d][qb][i] = 0.f;
  // row sums of P: ones x P^T on the MFMA, every register of a lane holds its
  // query's sum (of the same bf16 P values as the numerator)
  f32x16 acc_l[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc_l[qb][i] = 0.f;
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
  // running max floor: finite, so a row whose first tiles are all masked (in
  // descending order) gets p = 2^(-inf) = 0 there, not inf - inf
  float m_run[2] = {-1e30f, -1e30f};
  const int qpos0 = a.start_pos + q0 + FA_QW * wave;  // position of the wave's first query
  // tiles whose keys are all after every query of this wave are only moved, not used
  // Ascending: tiles whose keys are all after every query of this wave are only
  // moved, not used.  Descending: such tiles come first, and the wave runs
  // them masked (its SIMD would wait at the barriers anyway).
  const int nt_wave = desc ? nt_all : min(ntiles, (qpos0 + FA_QW - 1) / FA_KT + 1);

  f32x16 sA[2][2], sB[2][2];  // S^T [key block][query block] of two consecutive tiles
  u32x4 pA[4][2], pB[4][2];   // P^T [key step][query block] of two consecutive tiles

  // One pipeline step for tile t, all in one instruction stream:
  //   MFMA: S^T of tile t+1 (48, if QK) then O^T += V^T P^T of tile t-1 (32, if PV)
  //   VALU: softmax of tile t (mask, max, running max, exp, P^T pack, row sum),
  //         one slot after each MFMA
  // then the accumulator rescale for tile t's running max.  Tile t+1's k rows
  // and tile t-1's v rows are in LDS.
  auto step = [&](int t, f32x16 (&sc)[2][2], f32x16 (&sn)[2][2], u32x4 (&pc)[4][2], u32x4 (&pp)[4][2]) {
    // tile t+3's loads go out one every 8 MFMAs (a burst would stall the wave
    // on the memory pipeline)
    const TileSrc ts = tile_src(t + 3);
    const uint32_t kq = smem_addr + ((t + 1) % FA_NK) * FA_KSTAGE + kx;
    const uint32_t rq = smem_addr + ((t + 1) % FA_NK) * FA_KSTAGE + rx;
    const uint32_t vq = smem_addr + FA_VBASE + ((t + FA_NV - 1) % FA_NV) * FA_VSTAGE + vx;
    const int kt = key_tile(t);
    if (kt * FA_KT + FA_KT - 1 > qpos0) {
      // a tile on (or past) the diagonal: key kt*64 + 32 kb + 8 (i/4) + 4 hi + i%4
      // is masked for query qpos0 + 32 qb + l32 when 8 (i/4) + i%4 exceeds thr
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          fa_causal_mask(sc[kb][qb], qpos0 + 32 * qb + l32 - kt * FA_KT - 32 * kb - 4 * hi);
    }
    // MFMA order: 44 units of two MFMAs (query blocks 0, 1), interleaving
    // S^T of tile t+1 with O^T += V^T P^T of tile t-1 so the transposing
    // value reads and the key reads share the LDS evenly (fa_unit_kind).
    constexpr int NF = 40, NM = 88, NSTEP = NM;
    constexpr int FW = 3;  // fragments read ahead
    u32x4 fr[FW + 1];
    auto load_frag = [&](auto G) -> u32x4 {
      constexpr int u = fa_load_unit(decltype(G)::value);
      if constexpr (fa_unit_kind(u) == 'P') {
        constexpr int ks = u / 11, d = (u % 11 - 1) / 2;
        const uint32_t vb = (vq ^ (64 * d)) + ks * 16 * 256;
        const u32x2 lo = fa_tr16(vb), hv = fa_tr16(vb + 8 * 256);
        return u32x4{lo[0], lo[1], hv[0], hv[1]};
      } else {
        constexpr int f = fa_unit_q(u), kb = f / 12, s = f % 12;
        if constexpr (s < 8)
          return fa_lds16((kq ^ (32 * s)) + kb * 32 * 256);
        else
          return fa_lds16((rq ^ (32 * (s - 8))) + kb * 32 * 128);
      }
    };
    float mx[2] = {-INFINITY, -INFINITY}, mh[2], alpha[2], xa, xb, ea, eb;
    bool need[2];
    static_for<FW>([&](auto G) { fr[decltype(G)::value] = load_frag(G); });
    static_for<NSTEP>([&](auto J) {
      constexpr int j = decltype(J)::value;
      constexpr int u = j / 2, qb = j % 2;
      constexpr char kind = fa_unit_kind(u);
      if constexpr (kind != 'O' && qb == 0 && fa_unit_load(u) + FW < NF)
        fr[(fa_unit_load(u) + FW) % (FW + 1)] = load_frag(std::integral_constant<int, fa_unit_load(u) + FW>{});
      if constexpr (j % 8 == 4 && j / 8 < FA_DMA) dma_one(ts, j / 8);
      if constexpr (kind == 'P') {
        constexpr int ks = u / 11, d = (u % 11 - 1) / 2;
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
            : "+a"(acc[d][qb]) : "v"(fr[fa_unit_load(u) % (FW + 1)]), "v"(pp[ks][qb]));
      } else if constexpr (kind == 'O') {
        constexpr int ks = u / 11;
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc_l[qb]) : "v"(ones), "v"(pp[ks][qb]));
      } else {
        constexpr int f = fa_unit_q(u), kb = f / 12, s = f % 12;
        if constexpr (s == 0)
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
              : "=v"(sn[kb][qb]) : "v"(fr[fa_unit_load(u) % (FW + 1)]), "a"(qf[qb][s]));
        else
          asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
              : "+v"(sn[kb][qb]) : "v"(fr[fa_unit_load(u) % (FW + 1)]), "a"(qf[qb][s]));
      }
      // Softmax of tile t, one slot after each MFMA.  No instruction in a slot
      // uses a result from the same slot (the wave issues in order, so a wait
      // on a VALU result would also hold up the next MFMA).
      if constexpr (j < 16) {  // row max over the tile, two values per query block per slot
        constexpr int kb = j >> 3, i = 2 * (j & 7);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mx[qb] = fa_max3(mx[qb], sc[kb][qb][i], sc[kb][qb][i + 1]);
      } else if constexpr (j == 16) {  // the other half of each query's keys is in lane l ^ 32
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx[qb]), __float_as_uint(mx[qb]), false, false);
          mx[qb] = __uint_as_float(r[0]);
          mh[qb] = __uint_as_float(r[1]);
        }
      } else if constexpr (j == 17) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mx[qb] = fa_max3(mx[qb], mh[qb], mh[qb]);
      } else if constexpr (j == 18) {  // tile max in log2 units; the raise threshold
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          mx[qb] *= scale_log2;
          mh[qb] = m_run[qb] + FA_SLACK;
        }
      } else if constexpr (j == 19) {
        // running max, raised only when the tile max exceeds it by more than
        // FA_SLACK (p <= 2^8 stays exact in fp32); from the floor, the first
        // tile with a visible key raises it, with alpha = 2^(-1e30 - m) = 0
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) need[qb] = __any(mx[qb] > mh[qb]);
      } else if constexpr (j == 20) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mx[qb] = fa_max3(mx[qb], m_run[qb], m_run[qb]);
      } else if constexpr (j == 21) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) mh[qb] = need[qb] ? mx[qb] : m_run[qb];  // new running max
      } else if constexpr (j == 22) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) alpha[qb] = m_run[qb] - mh[qb];  // (exponentiated only when used)
      } else if constexpr (j == 23) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) m_run[qb] = mh[qb];
      }
      // score e (0..63, pair k = e/2, half e%2): x = s * scale - m at slot
      // 22 + e, its exponential at 23 + e, the pair's bf16 pack into P^T at
      // 25 + 2k.  One exponential per slot: v_exp_f32 issues at a quarter of
      // the VALU rate, and two in one slot outlasted the MFMA they shadow.
      if constexpr (j >= 25 && (j - 25) % 2 == 0 && (j - 25) / 2 < 32) {
        constexpr int k = (j - 25) / 2, qb = k >> 4, kb = (k >> 3) & 1, h2 = (k >> 2) & 1, e = k & 3;
        pc[2 * kb + h2][qb][e] = pack_bf16x2(ea, eb);
      }
      if constexpr (j >= 23 && j - 23 < 64) {
        if constexpr ((j - 23) % 2 == 0)
          ea = __builtin_amdgcn_exp2f(xa);
        else
          eb = __builtin_amdgcn_exp2f(xb);
      }
      if constexpr (j >= 22 && j - 22 < 64) {
        constexpr int sc_e = j - 22, k = sc_e / 2, qb = k >> 4, kb = (k >> 3) & 1, h2 = (k >> 2) & 1, e = k & 3;
        constexpr int i = 8 * h2 + 2 * e + (sc_e % 2);
        if constexpr (sc_e % 2 == 0)
          xa = __builtin_fmaf(sc[kb][qb][i], scale_log2, -mh[qb]);
        else
          xb = __builtin_fmaf(sc[kb][qb][i], scale_log2, -mh[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // P^T of tile t is consumed here, in this block: otherwise the compiler
    // sinks the whole softmax past the rescale branch into the next step's
    // block, where it runs as one burst between two MFMAs instead of in the
    // slots above
    asm volatile("" ::"v"(pc[0][0]), "v"(pc[0][1]), "v"(pc[1][0]), "v"(pc[1][1]), "v"(pc[2][0]), "v"(pc[2][1]),
                 "v"(pc[3][0]), "v"(pc[3][1]));
    // the accumulator now holds tiles <= t-1 at the old running max
    if (need[0] || need[1]) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) alpha[qb] = __builtin_amdgcn_exp2f(alpha[qb]);
      asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        if (need[qb]) {
#pragma unroll
          for (int d = 0; d < 4; ++d) fa_scale_tuple(acc[d][qb], alpha[qb]);
          fa_scale_tuple(acc_l[qb], alpha[qb]);
        }
      asm volatile("s_nop 4" ::: "memory");
    }
  };
  // O^T += V^T P^T for the wave's last tile (its v rows are still in LDS)
  auto pv_last = [&](int t, u32x4 (&pc)[4][2]) {
    const uint32_t vq = smem_addr + FA_VBASE + (t % FA_NV) * FA_VSTAGE + vx;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int ks = g >> 2, d = g & 3;
      const uint32_t vb = (vq ^ (64 * d)) + ks * 16 * 256;
      const u32x2 lo = fa_tr16(vb), hv = fa_tr16(vb + 8 * 256);
      const u32x4 vf = {lo[0], lo[1], hv[0], hv[1]};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[d][qb]) : "v"(vf), "v"(pc[ks][qb]));
      if (d == 3) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc_l[qb]) : "v"(ones), "v"(pc[ks][qb]));
      }
    }
  };
  // every wave waits for tile t+1, then the stages of tiles t-2 (k rows) and
  // t-3 (v rows) take tile t+3
  auto sync = [&]() {
    fa_wait_vmcnt<FA_DMA>();
    __syncthreads();
  };

  // prologue: S^T of tile 0.  The first step's value product runs on a
  // zeroed "tile -1" (the v stage tile 4 takes later) with P^T = 0.
#pragma unroll
  for (int i = 0; i < FA_VSTAGE / (256 * 16); ++i)
    *(u32x4*)(smem + FA_VBASE + (FA_NV - 1) * FA_VSTAGE + (i * 256 + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) pB[k][qb] = u32x4{0u, 0u, 0u, 0u};
  fa_wait_vmcnt<2 * FA_DMA>();
  __syncthreads();
#pragma unroll
  for (int f = 0; f < 24; ++f) {
    const int kb = f / 12, s = f % 12;
    const u32x4 kf = s < 8 ? fa_lds16(((smem_addr + kx) ^ (32 * s)) + kb * 32 * 256)
                           : fa_lds16(((smem_addr + rx) ^ (32 * (s - 8))) + kb * 32 * 128);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (s == 0)
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(sA[kb][qb]) : "v"(kf), "a"(qf[qb][s]));
      else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(sA[kb][qb]) : "v"(kf), "a"(qf[qb][s]));
    }
  }
  // wait states before VALU reads the MFMA results
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // A wave with an odd tile count runs one more, all of whose keys are after
  // its queries: fully masked, it adds nothing.  Every wave passes the same
  // number of barriers, one per tile step up to nt_all.
  const int nt_even = (nt_wave + 1) & ~1;
  int t = 0;
  for (; t < nt_even; t += 2) {
    sync();
    step(t, sA, sB, pA, pB);
    sync();
    step(t + 1, sB, sA, pB, pA);
  }
  pv_last(t - 1, pB);
  for (; t < nt_all; ++t) {
    sync();
    issue_tile(t + 3);
  }
  fa_wait_vmcnt<0>();  // tiles past the end still write LDS: drain them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]), "+a"(acc[2][0]),
                 "+a"(acc[2][1]), "+a"(acc[3][0]), "+a"(acc[3][1]), "+a"(acc_l[0]), "+a"(acc_l[1]));

  // ---- out[t][head][:] = O^T[:, t] / l.  Lane (l32, hi), tuple (d, qb),
  // register 4g + e: dim 32 d + 8 g + 4 hi + e of query 32 qb + l32; lanes l
  // and l + 32 trade halves (v_permlane32_swap) so each stores 8 whole dims.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int tq = q0 + FA_QW * wave + 32 * qb + l32;
    const float inv = 1.f / acc_l[qb][0];
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

// Persistent workgroups, one per CU (the LDS allows no second): workgroup g
// runs on XCD g % 8 and takes items of that XCD's contiguous range of work
// ids (head after head, each head's query groups longest first).  The P
// workgroups of an XCD take the range in rounds of P ids, in snake order
// (slot k takes id k of an even round and id P-1-k of an odd one): with P
// query groups per head, each pair of rounds gives every workgroup one long
// and one short item of equal total length, so the workgroups stay in step.
// Even rounds run their key tiles upward and odd rounds downward: all items
// of an even round start together and are at the same key tile at any
// moment; an odd-round item starts when its slot's even-round item ends,
// and counting down from its own top tile it, too, is at the same tile as
// every other odd-round item.  So the XCD's L2 holds the few tiles of at
// most two heads that all its workgroups are reading.  (One workgroup per
// item left each CU idle for a median 11.5 us between items, as the
// dispatcher did not hand the next workgroup to the CU just freed; and
// persistent rounds that all ran upward, the odd ones starting staggered,
// fetched 2.6 times the bytes from HBM.)
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fa_bf16_kernel(FaArgs a, int n_work) {
  const int G = (int)gridDim.x, g = (int)blockIdx.x, x = g % 8, k = g / 8;
  const int q = n_work / 8, r = n_work % 8;
  const int n_x = q + (x < r ? 1 : 0), base = x * q + min(x, r);  // this XCD's ids
  const int P = (G - x + 7) / 8;                                    // its workgroups
  bool first = true;
  for (int rd = 0; rd * P < n_x; ++rd) {
    const int i = rd * P + ((rd & 1) ? P - 1 - k : k);
    if (i >= n_x) continue;
    if (!first) __syncthreads();  // every wave is done with the previous item's LDS
    first = false;
    fa_item(a, base + i, (rd & 1) != 0);
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
    const int64_t slot = (int64_t)page * g.page_size + j % g.page_size;
    if (g.fp8) {
      // 656-byte rows: E4M3 codes of c^KV (scale 2^e per 128 values at byte
      // 640 + 4 tile), then k^R in bf16 from byte 512
      const unsigned char* r = (const unsigned char*)g.pool + slot * 656;
      if (c < 64) {
        const uint2 w = *reinterpret_cast<const uint2*>(r + 8 * c);
        const float sc = *reinterpret_cast<const float*>(r + 640 + 4 * (c >> 4));
        v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, sc, false));
        v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, sc, true));
        v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, sc, false));
        v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, sc, true));
      } else {
        v = *reinterpret_cast<const u32x4*>(r + 512 + 16 * (c - 64));
      }
    } else {
      v = *reinterpret_cast<const u32x4*>((const bf16*)g.pool + slot * g.row + 8 * c);
    }
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
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t grid = std::min<int64_t>(n, std::max(cus, 8));  // one workgroup per CU
  hipLaunchKernelGGL(fa_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, st, a, (int)n);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const GatherArgs& g, hipStream_t st) {
  const int64_t n = (int64_t)g.B * g.kv_end * (g.row / 8);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace mla
