// Dense projections of the MLA layer as batched GEMMs, C = A . B^T with bf16
// operands and fp32 accumulation on the MFMA (v_mfma_f32_16x16x32_bf16 in the
// large-tile kernel, v_mfma_f32_32x32x16_bf16 in the others).
//
// Uses (notes page "【论文解读】DeepSeek-V3", section 一(一)):
//   [c^KV_raw ; k^R_raw] = [W^DKV ; W^KR] h    (section 2 and the decoupled-RoPE
//                                             key of section 3; two weight
//                                             segments, one launch)
//   c^Q_raw = W^DQ h,  q^C = W^UQ c^Q,  q^R_raw = W^QR c^Q
//   q_lat_i = W_i^UK^T q^C_i   (absorption; B given as [K, N] = W_i^UK rows)
//   o_i = W_i^UV o_lat_i       (W^UV after the weighted sum of latents)
//   q^R = RoPE(W^QR c^Q)       (explicit prefill: the rotation in the output
//                               stage of the large-tile kernel)
//
// Three kernels by shape:
//  * gemm_big_kernel: at least 256 rows and enough tiles to fill the CUs
//    (the prefill projections): 256 x 256 / 256 x 192 tiles, see below.
//  * gemm_smallm_bf16_kernel: at most 256 rows, K <= 512 (decode projections).
//  * gemm_bf16_kernel: everything else, including B given [K, N].  Tiles
//    128 x 128 x 64, four waves in a 2 x 2 arrangement, each wave a 64 x 64
//    block of four 32 x 32 MFMA accumulators; A and B tiles staged through
//    double-buffered LDS (row stride 144 B: conflict-free 16-byte fragment
//    reads), the next K slice fetched into registers while the current one is
//    consumed; a weight given [K, N] (absorption) is transposed in registers
//    while staging.
// Ragged M and N are handled by buffer-resource bounds (out-of-range rows load
// as zero) and masked stores; K must be a multiple of 64 (32 for the
// large-tile kernel).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_plan.h"

namespace mla {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LSTR = BK * 2 + 16;        // bytes per tile row in LDS
constexpr int ABYTES = BM * LSTR, BBYTES = BN * LSTR;
constexpr int GSTAGE = ABYTES + BBYTES;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int32_t)(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// physical LDS row of tile row n (breaks 8-way conflicts of the transposed
// writes; a permutation within each aligned group of 8 rows)
__device__ __forceinline__ int prow(int n) { return n ^ ((n >> 3) & 7); }

template <bool B_KN, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * GSTAGE];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_n = (g.N + BN - 1) / BN;
  const int tn = blockIdx.x % tiles_n, tm = blockIdx.x / tiles_n;
  const int z = blockIdx.y;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16* A = (const bf16*)g.A + z * g.strideA;
  const bf16* B = (const bf16*)g.B + z * g.strideB;
  const bf16* B2 = g.B2 ? (const bf16*)g.B2 + z * g.strideB : nullptr;

  // --- staging assignment -------------------------------------------------
  // A: chunk c = tid + 256*i (i < 4): row c/8, k chunk c%8 (16 B each).
  // B (NK): same on the N rows.  B (KN): threads < 128 each own an 8 (k) x 8 (n)
  // block: k rows 8*(tid/16) .. +7, n columns 8*(tid%16) .. +7.
  const int rows_a = min(BM, g.M - m0);
  const __amdgpu_buffer_rsrc_t ra = rsrc(A + (int64_t)m0 * g.lda, (int64_t)(rows_a - 1) * g.lda * 2 + g.K * 2);
  // B rows r < split_local come from rb, the rest from rb2 (row r - split_local):
  // a tile straddling the W^DKV / W^KR boundary takes its upper rows from B2.
  __amdgpu_buffer_rsrc_t rb, rb2;
  int split_local = BN;
  if (!B_KN) {
    if (B2 && n0 >= g.n_split) {
      const int rows = min(BN, g.N - n0);
      rb = rsrc(B2 + (int64_t)(n0 - g.n_split) * g.ldb, (int64_t)(rows - 1) * g.ldb * 2 + g.K * 2);
    } else {
      const int lim = B2 ? g.n_split : g.N;
      const int rows = min(BN, lim - n0);
      rb = rsrc(B + (int64_t)n0 * g.ldb, (int64_t)(rows - 1) * g.ldb * 2 + g.K * 2);
    }
    rb2 = rb;
    if (B2 && n0 < g.n_split && n0 + BN > g.n_split) {
      split_local = g.n_split - n0;
      const int rows2 = min(BN - split_local, g.N - g.n_split);
      rb2 = rsrc(B2, (int64_t)(rows2 - 1) * g.ldb * 2 + g.K * 2);
    }
  } else {
    // [K, N] with leading dimension ldb; columns n0 .. n0+BN-1
    const int cols = min(BN, g.N - n0);
    rb = rsrc(B + n0, (int64_t)(g.K - 1) * g.ldb * 2 + cols * 2);
    rb2 = rb;
  }

  u32x4 sa[4], sb[8];
  auto load = [&](int kt) {
    const int kbyte = kt * BK * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
      sa[i] = bld16(ra, (int32_t)((int64_t)r * g.lda * 2 + kbyte + kc * 16));
    }
    if (!B_KN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        if (r < split_local)
          sb[i] = bld16(rb, (int32_t)((int64_t)r * g.ldb * 2 + kbyte + kc * 16));
        else
          sb[i] = bld16(rb2, (int32_t)((int64_t)(r - split_local) * g.ldb * 2 + kbyte + kc * 16));
      }
    } else if (tid < 128) {
      const int kb = tid >> 4, nb = tid & 15;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sb[e] = bld16(rb, (int32_t)((int64_t)(kt * BK + 8 * kb + e) * g.ldb * 2 + nb * 16));
    }
  };
  auto store = [&](int buf) {
    unsigned char* As = smem + buf * GSTAGE;
    unsigned char* Bs = As + ABYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
      st16(As + r * LSTR + kc * 16, sa[i]);
    }
    if (!B_KN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
        st16(Bs + prow(r) * LSTR + kc * 16, sb[i]);
      }
    } else if (tid < 128) {
      const int kb = tid >> 4, nb = tid & 15;
      u32x4 tr[8];
      transpose8x8(sb, tr);  // tr[d]: k = 8*kb .. 8*kb+7 of column n = 8*nb + d
#pragma unroll
      for (int d = 0; d < 8; ++d) st16(Bs + prow(8 * nb + d) * LSTR + kb * 16, tr[d]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = g.K / BK;
  load(0);
  store(0);
  if (nk > 1) load(1);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
    const unsigned char* As = smem + (kt & 1) * GSTAGE;
    const unsigned char* Bs = As + ABYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      u32x4 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const u32x4*)(As + (wm * 64 + 32 * i + l32) * LSTR + (16 * ks + 8 * hi) * 2);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const u32x4*)(Bs + prow(wn * 64 + 32 * j + l32) * LSTR + (16 * ks + 8 * hi) * 2);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      store((kt + 1) & 1);
      if (kt + 2 < nk) load(kt + 2);
    }
  }

  // --- epilogue: lane holds rows 8*(r/4) + 4*hi + r%4, column l32 of each block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + 32 * j + l32;
      if (col >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < g.M) {
          const int64_t o = z * g.strideC + (int64_t)row * g.ldc + col;
          if (OUT_BF16)
            ((bf16*)g.C)[o] = (bf16)acc[i][j][r];
          else
            ((float*)g.C)[o] = acc[i][j][r];
        }
      }
    }
}

// ---- large-tile GEMM (B given [N, K]) ---------------------------------------
// Output tile 256 x BN (BN = 256 or 192), four waves in a 2 x 2 arrangement,
// each wave a 128 x BN/2 block of 16 x 16 accumulators in AGPRs (8 x 8 or
// 8 x 6 of them), so each 16-byte fragment read from LDS feeds several MFMAs
// (an A fragment BN/32, a B fragment 8).  The 16 x 16 x 32 instruction does
// the work of half a 32 x 32 x 16 one in half the cycles, but on all CUs with
// random operands it sustains 14 % more FLOP/s (2.05 against 1.80 PFLOP/s),
// and this kernel ran 2-9 % faster with it than with 32 x 32 x 16 tiles.
// K moves in slices of 32 through a ring of four LDS stages
// filled by direct-to-LDS buffer loads (three slices in flight).  Each 64-byte
// tile row keeps its four 16-byte chunks at chunk ^ ((row >> 2) & 2).  The
// LDS (64 banks of 4 bytes, so 16 bank groups of 16 bytes) serves a 16-byte
// read in four passes of 16 lanes, two per half-wave, the half-wave's 4-lane
// groups split by the parity of the group index (lanes 0-3, 12-15, 20-27 in
// one pass, 4-11, 16-19, 28-31 in the other: measured pair by pair with a
// probe that times reads where only two lanes address different rows of one
// bank group).  A fragment read (lane (l16, q4): row l16, chunk q4) puts in
// one pass rows r, r + 12 of chunk q4 and rows r + 4, r + 8 of chunk q4 ^ 1
// (r < 4), and rows r, r + 4, r + 8, r + 12 share a bank group: the
// permutation sends those four reads to four different chunks.  With
// chunk ^ ((row >> 2) & 3) two of them met and every fragment read took
// twice the LDS cycles (bank-conflict stalls of 8-14 % of the kernel time
// were counted).  The loads apply the permutation on the global side.  The product is formed transposed
// (C^T = B A^T) so each lane holds four consecutive output columns; the output
// goes through LDS so that every store writes whole rows.
constexpr int GB_BM = 256, GB_BK = 32, GB_NST = 4, GB_GM = 4;
constexpr int GB_SK_BN = 192;  // column tile of the stream-K form
constexpr int GB_ROW = GB_BK * 2;  // bytes per tile row

// 16 bytes per lane from buffer offset voff + soff into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void gb_dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, int32_t voff, int32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(r), "s"(soff)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void gb_wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ u32x4 gb_lds16(uint32_t addr) {
  return *(const __attribute__((address_space(3))) u32x4*)addr;
}
template <typename T>
__device__ __forceinline__ const T* gb_uniform(const T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): every index
// a compile-time constant, so register arrays indexed by it stay in registers
template <typename F, int... J>
__device__ __forceinline__ void gb_static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void gb_static_for(F&& f) {
  gb_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int BN, bool OUT_BF16, bool ROPE = false, bool SK = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_big_kernel(GemmArgs g) {
  constexpr int A_BYTES = GB_BM * GB_ROW, B_BYTES = BN * GB_ROW, STG = A_BYTES + B_BYTES;
  constexpr int NI = 8;                        // 16-row MFMA tiles per wave (128 rows)
  constexpr int NJ = BN / 32;                  // 16-column MFMA tiles per wave (8 or 6)
  constexpr int NA = GB_BM / 16 / 4;           // A loads per wave per slice (4)
  constexpr int NB = BN / 16 / 4;              // B loads per wave per slice (4 or 3)
  constexpr int NLD = NA + NB;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GB_NST * STG];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_n = (g.N + BN - 1) / BN, tiles_m = (g.M + GB_BM - 1) / GB_BM;
  const int nk = g.K / GB_BK;
  const int64_t lda2 = g.lda * 2, ldb2 = g.ldb * 2;
  // Load i of wave w moves tile rows 16 (4 i + w) .. +15 (64 bytes each):
  // lane l writes LDS bytes 16 l of that 1 KB, i.e. row + l/4, slot l%4,
  // holding the row's logical chunk (l%4) ^ ((l/16) & 2).
  const int32_t va = (int32_t)((lane >> 2) * lda2) + 16 * ((lane & 3) ^ ((lane >> 4) & 2));
  const int32_t vb = (int32_t)((lane >> 2) * ldb2) + 16 * ((lane & 3) ^ ((lane >> 4) & 2));
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  // 16 x 16 x 32 MFMA fragments: lane (l16, q4) holds tile row R = base + l16
  // (16 rows per fragment), k 8 q4 .. 8 q4 + 7 of the slice, i.e. logical
  // chunk q4 of the row, stored at q4 ^ ((R >> 2) & 2); the row bases are
  // multiples of 16, so the XOR term is the same for every fragment.
  const int ra = wm * 128 + l16, rb = wn * (BN / 2) + l16;
  const uint32_t fa = ra * GB_ROW + 16 * (q4 ^ ((ra >> 2) & 2));            // + 16 i rows
  const uint32_t fb = A_BYTES + rb * GB_ROW + 16 * (q4 ^ ((rb >> 2) & 2));  // + 16 j rows
  u32x4 af[2][NI], bfr[2][NJ];  // fragments of two slices (the one in use, the next)
  f32x4 acc[NI][NJ];  // [m tile][n tile], C^T layout: lane holds columns 4 q4 .. +3 of row l16

  // Work of this workgroup.  Tile order: consecutive ids run on one XCD
  // (xcd_remap); within a group of GB_GM row tiles the column tile advances
  // every GB_GM ids, so the ~32 workgroups an XCD runs at once cover about
  // 4 x 8 tiles and share their A and B slices in that XCD's L2.
  // Stream-K (SK, batch 1): groups of tiles_n workgroups with consecutive ids
  // (so on one XCD, together) each take one column tile of the same rows; the
  // (row tile, k slice) units, k fastest, are cut into sk_wgs equal runs of
  // consecutive units, one per group.  A run covers the end of one row tile
  // and the start of the next (or more); each piece ("segment") writes fp32
  // partial sums of its tile to partial buffer p = this run's index minus
  // that of the run holding the row tile's first slice (sk_pstride elements
  // apart), and the consumer adds a row tile's partials (gemm_sk_parts).
  // The tiles_n workgroups of a group read the same rows of A at the same k,
  // so A comes from HBM about once.
  constexpr bool sk = SK;
  const int wgid = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int64_t U = (int64_t)tiles_m * nk, G = g.sk_wgs;
  const int grp = wgid / tiles_n;
  int64_t u = sk && grp < G ? (int64_t)grp * U / G : 0;
  const int64_t u_end = sk && grp < G ? (int64_t)(grp + 1) * U / G : 0;
  for (int seg = 0;; ++seg) {
  int tm, tn, ka, kend;
  int64_t coff;  // element offset of this segment's output
  if (sk) {
    if (u >= u_end) break;
    tm = (int)(u / nk);
    tn = wgid % tiles_n;
    ka = (int)(u % nk);
    kend = (int)min<int64_t>(nk, ka + (u_end - u));
    const int64_t first = (((int64_t)tm * nk + 1) * G - 1) / U;  // run holding the row tile's slice 0
    coff = (grp - first) * g.sk_pstride;
    u += kend - ka;
  } else {
    if (seg) break;
    const int group = wgid / (GB_GM * tiles_n), first_m = group * GB_GM;
    const int gsz = min(GB_GM, tiles_m - first_m), idx = wgid - group * GB_GM * tiles_n;
    tm = first_m + idx % gsz;
    tn = idx / gsz;
    ka = 0;
    kend = nk;
    coff = (int64_t)blockIdx.y * g.strideC;
  }
  const int ns = kend - ka;  // slices of this segment
  const int z = sk ? 0 : (int)blockIdx.y;
  const int m0 = tm * GB_BM, n0 = tn * BN;
  const unsigned char* A = (const unsigned char*)g.A + (int64_t)z * g.strideA * 2;
  const unsigned char* B = (const unsigned char*)g.B + (int64_t)z * g.strideB * 2;
  // One buffer resource per load, built once per tile: rows past M (or N) lie
  // outside it and load as zero; the slice's k offset goes in the scalar offset.
  __amdgpu_buffer_rsrc_t rsa[NA], rsb[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = 16 * (4 * i + wave);
    const int rows = max(0, min(16, g.M - m0 - row));
    const int32_t nbytes = rows > 0 ? (int32_t)((rows - 1) * lda2 + g.K * 2) : 0;
    rsa[i] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(gb_uniform(A + (int64_t)(m0 + row) * lda2)), (short)0, nbytes, 0x00020000);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + 16 * (4 * i + wave);  // first weight row of this load
    const unsigned char* p;
    int rows;
    if (g.B2 && n >= g.n_split) {
      p = (const unsigned char*)g.B2 + (int64_t)z * g.strideB * 2 + (int64_t)(n - g.n_split) * ldb2;
      rows = min(16, g.N - n);
    } else {
      p = B + (int64_t)n * ldb2;
      rows = min(16, (g.B2 ? g.n_split : g.N) - n);
    }
    const int32_t nbytes = rows > 0 ? (int32_t)((rows - 1) * ldb2 + g.K * 2) : 0;
    rsb[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(gb_uniform(p)), (short)0, nbytes,
                                               0x00020000);
  }
  // slice kt (past the end: the last slice again, into a stage nobody reads,
  // so every slice issues the same loads and the vmcnt bookkeeping stays uniform)
  // load n (< NA: A rows, else B rows) of slice kt
  auto issue_one = [&](int kt, int n) {
    const int32_t kb = __builtin_amdgcn_readfirstlane((ka + min(kt, ns - 1)) * GB_BK * 2);
    const uint32_t st = sbase + (kt % GB_NST) * STG;
    if (n < NA)
      gb_dma16(rsa[n], st + 16 * (4 * n + wave) * GB_ROW, va, kb);
    else
      gb_dma16(rsb[n - NA], st + A_BYTES + 16 * (4 * (n - NA) + wave) * GB_ROW, vb, kb);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int n = 0; n < NLD; ++n) issue_one(kt, n);
  };

#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.f;

  issue(0);
  issue(1);
  issue(2);
  gb_wait_vmcnt<2 * NLD>();
  __syncthreads();
  {
#pragma unroll
    for (int i = 0; i < NI; ++i) af[0][i] = gb_lds16(sbase + fa + i * 16 * GB_ROW);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[0][j] = gb_lds16(sbase + fb + j * 16 * GB_ROW);
  }
  // One slice: NI x NJ MFMAs on fragment set `set` (slice kt).  Halfway, the
  // barrier (slice kt+1 has landed everywhere; every wave read slice kt-1's
  // stage into registers during slice kt-2); the second half reads slice
  // kt+1's fragments into the other set and spreads slice kt+3's loads over
  // its MFMAs (a burst would hold up the MFMA issue).
  constexpr int NM = NI * NJ, HALF = NM / 2;
  auto slice = [&](const int kt, auto set_tag) __attribute__((always_inline)) {
    constexpr int set = decltype(set_tag)::value;
    const uint32_t sn = sbase + ((kt + 1) % GB_NST) * STG;
    gb_static_for<NM>([&](auto M) __attribute__((always_inline)) {
      constexpr int m = decltype(M)::value, i = m / NJ, j = m % NJ;
      if constexpr (m == HALF) {
        gb_wait_vmcnt<NLD>();
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(bfr[set][j]), "v"(af[set][i]));
      if constexpr (m >= HALF) {
        constexpr int h = m - HALF;  // one fragment of slice kt+1 after each of the first NI + NJ MFMAs
        if constexpr (h < NI) af[set ^ 1][h] = gb_lds16(sn + fa + h * 16 * GB_ROW);
        else if constexpr (h < NI + NJ) bfr[set ^ 1][h - NI] = gb_lds16(sn + fb + (h - NI) * 16 * GB_ROW);
#pragma unroll
        for (int n = 0; n < NLD; ++n)
          if (n * HALF / NLD == h) issue_one(kt + 3, n);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the MFMA / load interleave as written
    });
  };
  // (pairs of slices, so the fragment sets are compile-time indices)
  int kt = 0;
  for (; kt + 1 < ns; kt += 2) {
    slice(kt, std::integral_constant<int, 0>{});
    slice(kt + 1, std::integral_constant<int, 1>{});
  }
  if (kt < ns) slice(kt, std::integral_constant<int, 0>{});
  gb_wait_vmcnt<0>();  // the empty slices' loads still write LDS
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // Output through LDS, one wave's 128 x BN/2 block at a time per wave-private
  // quarter of the stage memory, so every store instruction writes whole rows: lane (l16, q4)
  // of acc[i][j] holds row 16 i + l16, columns 16 j + 4 q4 .. +3.  The block
  // goes through in passes of PR rows.  Rows of 16 or 32
  // chunks (256 columns) keep 16-byte chunk c at c ^ (row % CPR); rows of 12
  // or 24 chunks (192 columns) are staged with one spare chunk per row (an
  // odd stride in chunks), so the 16 rows one write pass covers fall in 16
  // different bank groups with no permutation.
  __syncthreads();  // every wave is done with the k-slice stages
  constexpr int ES = OUT_BF16 ? 2 : 4;                 // output element bytes
  constexpr int CPR = (BN / 2) * ES / 16;              // chunks per row (16 / 12 or 32 / 24)
  constexpr bool POW2 = (CPR & (CPR - 1)) == 0;
  constexpr int RB = (CPR + (POW2 ? 0 : 1)) * 16;      // staged row stride in bytes
  constexpr int PR = 32768 / RB >= 128 ? 128 : 64;     // rows per pass (whole 16-row tiles)
  // staged position of chunk c of row r, and its inverse
  const auto perm = [](int c, int r) { return POW2 ? c ^ (r & (CPR - 1)) : c; };
  const auto iperm = [](int p, int r) { return POW2 ? p ^ (r & (CPR - 1)) : p; };
  constexpr int EREG = GB_NST * STG / 4;  // each wave's share of the stage memory
  static_assert(PR * RB <= EREG, "staging pass exceeds the wave's LDS share");
  const uint32_t ew = sbase + wave * EREG;
  const int col0 = n0 + (BN / 2) * wn;
  unsigned char* cbase = (unsigned char*)g.C + coff * ES;
#pragma unroll
  for (int pass = 0; pass < 128 / PR; ++pass) {
#pragma unroll
    for (int ii = 0; ii < PR / 16; ++ii) {
      const int i = pass * (PR / 16) + ii;
      const int r = 16 * ii + l16;  // row within the pass
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 1; ++q) {
          const f32x4& t = acc[i][j];
          const int c = (16 * j + 4 * q4) * ES;  // byte column within the row
          if (OUT_BF16) {
            float x0 = t[0], x1 = t[1], x2 = t[2], x3 = t[3];
            if constexpr (ROPE) {
              // the four columns are two whole pairs (2p, 2p+1), (2p+2, 2p+3)
              const int row = m0 + 128 * wm + 16 * i + l16, col = col0 + 16 * j + 4 * q4;
              const int pr = (col % g.rope_d) >> 1;
              const f32x4 cs = *reinterpret_cast<const f32x4*>(
                  g.rope_cs + ((int64_t)(row % g.rope_rows) * (g.rope_d >> 1) + pr) * 2);
              const float y0 = cs[0] * x0 - cs[1] * x1, y1 = cs[1] * x0 + cs[0] * x1;
              const float y2 = cs[2] * x2 - cs[3] * x3, y3 = cs[3] * x2 + cs[2] * x3;
              x0 = y0; x1 = y1; x2 = y2; x3 = y3;
            }
            const u32x2 v = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
            const uint32_t addr = ew + r * RB + (perm(c >> 4, r) << 4) + (c & 15);
            *(__attribute__((address_space(3))) u32x2*)addr = v;
          } else {
            const f32x4 v = t;
            const uint32_t addr = ew + r * RB + (perm(c >> 4, r) << 4);
            *(__attribute__((address_space(3))) f32x4*)addr = v;
          }
        }
    }
    // (a wave reads back only its own writes: LDS ops of one wave complete in order)
    // A row takes LPR lanes (CPR rounded up to whole 16-lane passes): lane l
    // reads chunk position l % LPR of staged row l / LPR, so each pass reads
    // contiguous bytes of one row; with 12 or 24 chunks per row 4 or 8 lanes
    // of each row's last pass idle
    constexpr int LPR = (CPR + 15) / 16 * 16;
    constexpr int RSTEP = 64 / LPR;  // rows per read instruction
#pragma unroll 4
    for (int rr = 0; rr < PR; rr += RSTEP) {
      const int r = rr + lane / LPR, pos = lane % LPR;
      if (pos >= CPR || r >= PR) continue;
      const u32x4 v = gb_lds16(ew + r * RB + pos * 16);
      const int row = m0 + 128 * wm + pass * PR + r;
      const int col = col0 + (iperm(pos, r) * 16) / ES;
      if (row < g.M && col < g.N) *reinterpret_cast<u32x4*>(cbase + ((int64_t)row * g.ldc + col) * ES) = v;
    }
  }
  __syncthreads();  // every wave has read back its staging before the next segment's loads
  }
}

// fp32 SIMT GEMM for small shapes: 16 x 16 output tile per 256 threads.
template <bool B_KN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[16][17], Bs[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int tiles_n = (g.N + 15) / 16;
  const int n0 = (blockIdx.x % tiles_n) * 16, m0 = (blockIdx.x / tiles_n) * 16;
  const int z = blockIdx.y;
  const float* A = (const float*)g.A + z * g.strideA;
  const float* B = (const float*)g.B + z * g.strideB;
  const float* B2 = g.B2 ? (const float*)g.B2 + z * g.strideB : nullptr;
  float accv = 0.f;
  for (int k0 = 0; k0 < g.K; k0 += 16) {
    const int m = m0 + ty, k = k0 + tx;
    As[ty][tx] = (m < g.M && k < g.K) ? A[(int64_t)m * g.lda + k] : 0.f;
    const int n = n0 + ty;  // B tile stored [n][k]
    float bv = 0.f;
    if (n < g.N && k < g.K) {
      if (B_KN)
        bv = B[(int64_t)k * g.ldb + n];
      else if (B2 && n >= g.n_split)
        bv = B2[(int64_t)(n - g.n_split) * g.ldb + k];
      else
        bv = B[(int64_t)n * g.ldb + k];
    }
    Bs[ty][tx] = bv;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) accv += As[ty][kk] * Bs[tx][kk];
    __syncthreads();
  }
  const int m = m0 + ty, n = n0 + tx;
  if (m < g.M && n < g.N) ((float*)g.C)[z * g.strideC + (int64_t)m * g.ldc + n] = accv;
}


// ---------------------------------------------------------------------------
// Small-M batched GEMM (decode: M = query rows <= 256 per head, K <= 512): one
// workgroup per (64-column block, batch entry, 64-row block) holds the whole
// K extent of its A and B tiles in LDS, so it makes one round of loads instead of a
// pipeline of K slices, and the many small workgroups keep enough loads in
// flight.  Four waves in a 2 x 2 arrangement of 32 x 32 MFMA tiles.  The
// output tile is staged in LDS and written with 16-byte stores.
constexpr int SM_BM = 64, SM_BN = 64;

template <bool B_KN, int KMAX, bool PLAN>
__global__ __launch_bounds__(256) void gemm_smallm_bf16_kernel(GemmArgs g, PlanJob pj) {
  if constexpr (PLAN) {
    // columns past the batch pad the grid width to a multiple of 8 (so each
    // batch entry keeps its XCD); the first of them builds the attention plan
    if ((int)blockIdx.x >= g.batch) {
      if ((int)blockIdx.x == g.batch && blockIdx.y == 0 && blockIdx.z == 0)
        plan_body(pj.a, pj.plan, pj.target_items, pj.min_chunk, pj.max_chunk);
      return;
    }
  }
  constexpr int RS = KMAX * 2 + 16;  // LDS row stride in bytes (16-byte pad: conflict-free fragment reads)
  __shared__ __attribute__((aligned(16))) unsigned char sa[SM_BM * RS];
  __shared__ __attribute__((aligned(16))) unsigned char sb[SM_BN * RS];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  // grid (batch, column blocks, row blocks of 64): consecutive workgroups
  // (which the dispatcher deals round-robin to the XCDs) take different batch
  // entries, so the column and row blocks of one batch entry share an XCD and
  // its L2 copies of the A and B tiles
  const int n0 = blockIdx.y * SM_BN, z = blockIdx.x, m0 = blockIdx.z * SM_BM;
  const int Mb = min(SM_BM, g.M - m0);  // rows of this block
  const int K = g.K, kc = K / 8;  // 16-byte chunks per row
  const bf16* A = (const bf16*)g.A + z * g.strideA + (int64_t)m0 * g.lda;
  const bf16* B = (const bf16*)g.B + z * g.strideB;

  // All loads are issued before any LDS store so they are in flight together.
  constexpr int PER = SM_BM * (KMAX / 8) / 256;  // 16-byte chunks per thread and operand
  // A rows past M load as zero
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, (int64_t)(Mb - 1) * g.lda * 2 + K * 2);
  u32x4 va[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i, r = c / kc, k8 = c % kc;
    if (c < SM_BM * kc) va[i] = bld16(ra, (int32_t)((int64_t)r * g.lda * 2 + k8 * 16));
  }
  if (!B_KN) {  // B given [N, K]: rows of the column block
    const int rows = min(SM_BN, g.N - n0);
    const __amdgpu_buffer_rsrc_t rb = rsrc(B + (int64_t)n0 * g.ldb, (int64_t)(rows - 1) * g.ldb * 2 + K * 2);
    u32x4 vb[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i, r = c / kc, k8 = c % kc;
      if (c < SM_BN * kc) vb[i] = bld16(rb, (int32_t)((int64_t)r * g.ldb * 2 + k8 * 16));
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i, r = c / kc, k8 = c % kc;
      if (c < SM_BN * kc) *(u32x4*)(sb + r * RS + k8 * 16) = vb[i];
    }
  } else {  // B given [K, N]: 8 x 8 blocks transposed in registers to [n][k]
    const __amdgpu_buffer_rsrc_t rb = rsrc(B + n0, (int64_t)(K - 1) * g.ldb * 2 + (int64_t)min(SM_BN, g.N - n0) * 2);
    constexpr int BPER = ((KMAX / 8) * (SM_BN / 8) + 255) / 256;  // 8 x 8 blocks per thread
    u32x4 in[BPER][8];
#pragma unroll
    for (int q = 0; q < BPER; ++q) {
      const int blk = tid + 256 * q, kb = blk / (SM_BN / 8), nb = blk % (SM_BN / 8);
      if (blk < kc * (SM_BN / 8)) {
#pragma unroll
        for (int r = 0; r < 8; ++r) in[q][r] = bld16(rb, (int32_t)((int64_t)(8 * kb + r) * g.ldb * 2 + nb * 16));
      }
    }
#pragma unroll
    for (int q = 0; q < BPER; ++q) {
      const int blk = tid + 256 * q, kb = blk / (SM_BN / 8), nb = blk % (SM_BN / 8);
      if (blk < kc * (SM_BN / 8)) {
        u32x4 out[8];
        transpose8x8(in[q], out);
#pragma unroll
        for (int c = 0; c < 8; ++c) *(u32x4*)(sb + (8 * nb + c) * RS + kb * 16) = out[c];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i, r = c / kc, k8 = c % kc;
    if (c < SM_BM * kc) *(u32x4*)(sa + r * RS + k8 * 16) = va[i];
  }
  __syncthreads();

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const unsigned char* pa = sa + (32 * wm + l32) * RS + 16 * hi;
  const unsigned char* pb = sb + (32 * wn + l32) * RS + 16 * hi;
#pragma unroll 8
  for (int s = 0; s < K / 16; ++s) acc = mfma32(*(const u32x4*)(pa + 32 * s), *(const u32x4*)(pb + 32 * s), acc);
  __syncthreads();  // the A tile's LDS is reused for the output tile

  // lane l, register i: row 32 wm + 8 (i/4) + 4 hi + i%4, column 32 wn + l32
  constexpr int CS = SM_BN * 2 + 16;
  bf16* sc = (bf16*)sa;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    sc[(32 * wm + 8 * (i >> 2) + 4 * hi + (i & 3)) * (CS / 2) + 32 * wn + l32] = (bf16)acc[i];
  __syncthreads();
  bf16* C = (bf16*)g.C + z * g.strideC + (int64_t)m0 * g.ldc;
  for (int c = tid; c < SM_BM * (SM_BN / 8); c += 256) {
    const int r = c / (SM_BN / 8), c8 = c % (SM_BN / 8);
    if (r < Mb && n0 + 8 * c8 < g.N)
      *(u32x4*)(C + (int64_t)r * g.ldc + n0 + 8 * c8) = *(const u32x4*)(sa + r * CS + c8 * 16);
  }
}

}  // namespace

namespace {
constexpr int SM_MAX_ROWS = 4 * SM_BM;  // up to 4 row blocks
bool smallm_form(const GemmArgs& g) {
  return g.M <= SM_MAX_ROWS && g.K <= 512 && g.K % 64 == 0 && g.N % 8 == 0 && g.out_bf16 && !g.B2;
}

template <bool PLAN>
void launch_smallm(const GemmArgs& g, const PlanJob& pj, hipStream_t st) {
  const unsigned gx = PLAN ? (unsigned)((g.batch + 1 + 7) / 8 * 8) : (unsigned)g.batch;
  dim3 grid(gx, (unsigned)((g.N + SM_BN - 1) / SM_BN), (unsigned)((g.M + SM_BM - 1) / SM_BM));
  if (g.K <= 128) {
    if (g.b_kn)
      hipLaunchKernelGGL((gemm_smallm_bf16_kernel<true, 128, PLAN>), grid, dim3(256), 0, st, g, pj);
    else
      hipLaunchKernelGGL((gemm_smallm_bf16_kernel<false, 128, PLAN>), grid, dim3(256), 0, st, g, pj);
  } else {
    if (g.b_kn)
      hipLaunchKernelGGL((gemm_smallm_bf16_kernel<true, 512, PLAN>), grid, dim3(256), 0, st, g, pj);
    else
      hipLaunchKernelGGL((gemm_smallm_bf16_kernel<false, 512, PLAN>), grid, dim3(256), 0, st, g, pj);
  }
}
}  // namespace

namespace {
// The large-tile kernel: B given [N, K], 16-byte aligned rows, K a multiple of
// 32, whole 4-column output groups, and enough rows to fill its 256-row tiles.
bool bigtile_form(const GemmArgs& g) {
  const auto al16 = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
  const int cw = g.out_bf16 ? 8 : 4;  // output elements per 16-byte store
  return !g.b_kn && g.M >= GB_BM && g.K % GB_BK == 0 && g.N % cw == 0 && g.ldc % cw == 0 && g.lda % 8 == 0 &&
         g.ldb % 8 == 0 && g.strideA % 8 == 0 && g.strideB % 8 == 0 && g.strideC % cw == 0 && al16(g.A) &&
         al16(g.B) && al16(g.C) && (!g.B2 || (al16(g.B2) && g.n_split % 16 == 0)) &&
         (int64_t)15 * g.lda * 2 + g.K * 2 < (1LL << 31) && (int64_t)15 * g.ldb * 2 + g.K * 2 < (1LL << 31);
}
template <int BN, bool ROPE = false>
void launch_big(const GemmArgs& g, hipStream_t st) {
  const unsigned tiles = (unsigned)(((g.M + GB_BM - 1) / GB_BM) * ((g.N + BN - 1) / BN));
  dim3 grid(tiles, (unsigned)g.batch);
  if (ROPE)
    hipLaunchKernelGGL((gemm_big_kernel<BN, true, true>), grid, dim3(256), 0, st, g);
  else if (g.out_bf16)
    hipLaunchKernelGGL((gemm_big_kernel<BN, true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BN, false>), grid, dim3(256), 0, st, g);
}
}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (smallm_form(g)) {
    launch_smallm<false>(g, PlanJob{}, st);
    return hipGetLastError();
  }
  if (bigtile_form(g)) {
    // the column tile (256 or 192) that keeps more CUs busy over the launch's
    // rounds of 256 workgroups; too few tiles for either: the 128 x 128 kernel
    const auto fill = [&](int bn) {
      const int64_t t = (int64_t)((g.M + GB_BM - 1) / GB_BM) * ((g.N + bn - 1) / bn) * g.batch;
      const double useful = (double)g.M * g.N * g.batch / ((double)t * GB_BM * bn);
      return std::make_pair(t, useful * (double)t / (double)(((t + 255) / 256) * 256));
    };
    const auto f256 = fill(256), f192 = fill(192);
    if (std::max(f256.first, f192.first) >= 128) {
      if (f192.second > f256.second + 0.02)
        launch_big<192>(g, st);
      else
        launch_big<256>(g, st);
      return hipGetLastError();
    }
  }
  const unsigned tiles = (unsigned)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  dim3 grid(tiles, (unsigned)g.batch);
  if (g.b_kn) {
    if (g.out_bf16)
      hipLaunchKernelGGL((gemm_bf16_kernel<true, true>), grid, dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<true, false>), grid, dim3(256), 0, st, g);
  } else {
    if (g.out_bf16)
      hipLaunchKernelGGL((gemm_bf16_kernel<false, true>), grid, dim3(256), 0, st, g);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<false, false>), grid, dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_streamk(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.batch != 1 || g.out_bf16 || g.sk_wgs <= 0 || !bigtile_form(g)) return hipErrorNotSupported;
  const unsigned wgs = (unsigned)(g.sk_wgs * ((g.N + GB_SK_BN - 1) / GB_SK_BN));
  hipLaunchKernelGGL((gemm_big_kernel<GB_SK_BN, false, false, true>), dim3(wgs), dim3(256), 0, st, g);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_rope(const GemmArgs& g, hipStream_t st) {
  // whole pairs per 4-column group, whole 256-column tiles of heads, and a
  // 16-byte aligned cos/sin table
  if (g.M <= 0 || g.N <= 0 || g.batch != 1 || !g.out_bf16 || !g.rope_cs || g.rope_rows <= 0 || g.rope_d <= 0 ||
      g.rope_d % 4 != 0 || 256 % g.rope_d != 0 || g.N % 256 != 0 || ((uintptr_t)g.rope_cs & 15) != 0 ||
      !bigtile_form(g))
    return hipErrorNotSupported;
  launch_big<256, true>(g, st);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_plan(const GemmArgs& g, const PlanJob& p, hipStream_t st) {
  if (g.M > 0 && g.N > 0 && g.batch > 0 && smallm_form(g)) {
    launch_smallm<true>(g, p, st);
    return hipGetLastError();
  }
  hipError_t e = launch_attn_plan(p.a, p.plan, p.target_items, p.min_chunk, p.max_chunk, st);
  if (e != hipSuccess) return e;
  return launch_gemm_bf16(g, st);
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const unsigned tiles = (unsigned)(((g.M + 15) / 16) * ((g.N + 15) / 16));
  dim3 grid(tiles, (unsigned)g.batch);
  if (g.b_kn)
    hipLaunchKernelGGL((gemm_f32_kernel<true>), grid, dim3(256), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<false>), grid, dim3(256), 0, st, g);
  return hipGetLastError();
}

}  // namespace mla
