// Dense projections of the MLA layer as batched GEMMs, C = A . B^T with bf16
// operands and fp32 accumulation on v_mfma_f32_32x32x16_bf16.
//
// Uses (notes page "【论文解读】DeepSeek-V3", section 一(一)):
//   [c^KV_raw ; k^R_raw] = [W^DKV ; W^KR] h    (section 2 and the decoupled-RoPE
//                                             key of section 3; two weight
//                                             segments, one launch)
//   c^Q_raw = W^DQ h,  q^C = W^UQ c^Q,  q^R_raw = W^QR c^Q
//   q_lat_i = W_i^UK^T q^C_i   (absorption; B given as [K, N] = W_i^UK rows)
//   o_i = W_i^UV o_lat_i       (W^UV after the weighted sum of latents)
//
// Tiles: 128 x 128 x 64, four waves in a 2 x 2 arrangement, each wave a
// 64 x 64 block of four 32 x 32 MFMA accumulators.  A and B tiles are staged
// through double-buffered LDS (row stride 144 B: conflict-free 16-byte
// fragment reads); the next K slice is fetched into registers while the
// current one is consumed.  A weight given [K, N] (absorption) is transposed
// in registers while staging.  Ragged M and N are handled by buffer-resource
// bounds (out-of-range rows load as zero) and masked stores; K must be a
// multiple of 64.
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
  const bf16* B2 = (const bf16*)g.B2;

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
  const float* B2 = (const float*)g.B2;
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
// Small-M batched GEMM (decode: M = query rows <= 64 per head, K <= 512): one
// workgroup per (64-column block, batch entry) holds the whole K extent of
// its A and B tiles in LDS, so it makes one round of loads instead of a
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
      if ((int)blockIdx.x == g.batch && blockIdx.y == 0)
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
  // grid (batch, column blocks): consecutive workgroups (which the dispatcher
  // deals round-robin to the XCDs) take different batch entries, so the column
  // blocks of one batch entry share an XCD and its L2 copy of the A tile
  const int n0 = blockIdx.y * SM_BN, z = blockIdx.x;
  const int K = g.K, kc = K / 8;  // 16-byte chunks per row
  const bf16* A = (const bf16*)g.A + z * g.strideA;
  const bf16* B = (const bf16*)g.B + z * g.strideB;

  // All loads are issued before any LDS store so they are in flight together.
  constexpr int PER = SM_BM * (KMAX / 8) / 256;  // 16-byte chunks per thread and operand
  // A rows past M load as zero
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, (int64_t)(g.M - 1) * g.lda * 2 + K * 2);
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
  bf16* C = (bf16*)g.C + z * g.strideC;
  for (int c = tid; c < SM_BM * (SM_BN / 8); c += 256) {
    const int r = c / (SM_BN / 8), c8 = c % (SM_BN / 8);
    if (r < g.M && n0 + 8 * c8 < g.N)
      *(u32x4*)(C + (int64_t)r * g.ldc + n0 + 8 * c8) = *(const u32x4*)(sa + r * CS + c8 * 16);
  }
}

}  // namespace

namespace {
bool smallm_form(const GemmArgs& g) {
  return g.M <= SM_BM && g.K <= 512 && g.K % 64 == 0 && g.N % 8 == 0 && g.out_bf16 && !g.B2;
}

template <bool PLAN>
void launch_smallm(const GemmArgs& g, const PlanJob& pj, hipStream_t st) {
  const unsigned gx = PLAN ? (unsigned)((g.batch + 1 + 7) / 8 * 8) : (unsigned)g.batch;
  dim3 grid(gx, (unsigned)((g.N + SM_BN - 1) / SM_BN));
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

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (smallm_form(g)) {
    launch_smallm<false>(g, PlanJob{}, st);
    return hipGetLastError();
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
