// Element-wise parts of the MLA layer: the cache append (RMSNorm of c^KV,
// RoPE of k^R, paged scatter), the RMSNorm of c^Q and RoPE of q^R.
//
// Definitions (notes page "【论文解读】DeepSeek-V3"):
//  * RMSNorm after each compressed latent (section 二(二)1):
//      y = x / sqrt(mean(x^2) + eps) * g
//  * RoPE (section 一(一)3): each adjacent pair (x_2p, x_2p+1) is rotated by
//    the 2x2 block [[cos, -sin], [sin, cos]] at angle pos * theta_p, with
//    theta_p = base^(-2p/d_rope) (the frequency formula of the hnwysp.cn
//    digest, section 4.3).  Angles are formed and reduced in double precision:
//    at position 131072 a float angle would already be off by ~1e-2 rad.
//  * YaRN (section 三(二)3, the long-context extension, with the method's
//    meaning from the YaRN paper it points to): when yarn_s > 1 each theta_p
//    is interpolated by yarn_s where the pair turns fewer than alpha times
//    over the original window, kept where it turns more than beta times, and
//    ramped linearly between.
//  * Only [c^KV ; k^R] is cached per token (end of section 一(一)3); token p
//    of sequence b lives at slot p % page_size of page block_table[b][p / page_size].
#include <math.h>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int FLAG_BAD_PAGE = 1, FLAG_BAD_POS = 2, FLAG_BAD_SEQ = 8;

__device__ __forceinline__ void rope_cos_sin(int pos, int p, int d_rope, const RopeParams& rp, float& c, float& s) {
  double theta = pow((double)rp.base, -2.0 * (double)p / (double)d_rope);
  if (rp.yarn_s > 1.f) {
    const double r = (double)rp.yarn_orig * theta / (2.0 * M_PI);
    const double g = fmin(1.0, fmax(0.0, (r - (double)rp.yarn_alpha) / ((double)rp.yarn_beta - (double)rp.yarn_alpha)));
    theta = (1.0 - g) * theta / (double)rp.yarn_s + g * theta;
  }
  const double ang = (double)pos * theta;
  double sd, cd;
  sincos(ang, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

template <typename T>
__device__ __forceinline__ float ld_as_f32(const void* p, int64_t i) {
  return to_f32(((const T*)p)[i]);
}

// Partial products that make up input column col of token i: one, or those
// of a stream-K product (part_stride elements apart).
__device__ __forceinline__ int n_parts(const AppendArgs& a, int i, int col) {
  (void)col;  // every column tile of a row tile has the same partials
  if (!a.part_stride || !a.sk_wgs) return 1;
  const int64_t U = (int64_t)((a.n + GEMM_SK_BM - 1) / GEMM_SK_BM) * a.sk_nk;
  return gemm_sk_parts(i / GEMM_SK_BM, a.sk_nk, U, a.sk_wgs);
}

// One wave per appended token.
template <typename TIN, typename TOUT>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  int b, pos;
  if (a.seq_idx) {
    b = a.seq_idx[i];
    pos = a.pos[i];
  } else {
    b = i / a.L;
    pos = a.start_pos + i % a.L;
  }
  if (b < 0 || b >= a.n_seqs) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_SEQ);
    return;
  }
  const int pidx = pos >= 0 ? pos / a.page_size : -1;
  if (pidx < 0 || pidx >= a.max_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_POS);
    return;
  }
  const int page = a.block_table[(int64_t)b * a.max_pages + pidx];
  if (page < 0 || (int64_t)page >= a.num_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_PAGE);
    return;
  }
  const int row = a.d_c + a.d_rope;
  TOUT* dst = (TOUT*)a.pool + ((int64_t)page * a.page_size + pos % a.page_size) * row;
  const int64_t ci = (int64_t)i * a.ld_ckv, ki = (int64_t)i * a.ld_kr;
  // the projection, as one product or the sum of its partial products
  // (column col of the product: latent dims, then the d_rope of k^R)
  const auto in = [&](const void* p, int64_t o, int col) {
    float x = ld_as_f32<TIN>(p, o);
    const int np = n_parts(a, i, col);
    for (int q = 1; q < np; ++q) x += ld_as_f32<TIN>(p, o + q * a.part_stride);
    return x;
  };

  // RMSNorm of the latent
  float ss = 0.f;
  for (int d = lane; d < a.d_c; d += 64) {
    const float x = in(a.ckv, ci + d, d);
    ss += x * x;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)a.d_c + a.eps);
  for (int d = lane; d < a.d_c; d += 64) {
    const float x = in(a.ckv, ci + d, d);
    const float g = ld_as_f32<TOUT>(a.g_kv, d);
    dst[d] = from_f32<TOUT>(x * inv * g);
  }
  // RoPE of the shared decoupled key
  for (int p = lane; p < a.d_rope / 2; p += 64) {
    float c, s;
    if (a.rope_cs) {
      const float* cs = a.rope_cs + ((int64_t)(i % a.L) * (a.d_rope / 2) + p) * 2;
      c = cs[0];
      s = cs[1];
    } else {
      rope_cos_sin(pos, p, a.d_rope, a.rope, c, s);
    }
    const float x0 = in(a.kr, ki + 2 * p, a.d_c + 2 * p), x1 = in(a.kr, ki + 2 * p + 1, a.d_c + 2 * p + 1);
    dst[a.d_c + 2 * p] = from_f32<TOUT>(c * x0 - s * x1);
    dst[a.d_c + 2 * p + 1] = from_f32<TOUT>(s * x0 + c * x1);
  }
}

// The same for a bf16 cache with the V3 widths (d_c = 512, d_rope = 64),
// four tokens per workgroup (one per wave) and 16-byte accesses: lane l
// holds dims 8l .. 8l+7 of the latent (two 16-byte loads of fp32 input per
// partial, one of bf16 input) and writes them with one 16-byte store; lanes
// 0 .. 31 rotate pair l of k^R.
template <typename TIN>
__device__ __forceinline__ void load8(const void* p, int64_t o, float (&y)[8]) {
  if constexpr (sizeof(TIN) == 4) {
    const f32x4 u = *reinterpret_cast<const f32x4*>((const float*)p + o);
    const f32x4 v = *reinterpret_cast<const f32x4*>((const float*)p + o + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[k] = u[k];
      y[4 + k] = v[k];
    }
  } else {
    const u32x4 u = *reinterpret_cast<const u32x4*>((const bf16*)p + o);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[2 * k] = bf16_lo(u[k]);
      y[2 * k + 1] = bf16_hi(u[k]);
    }
  }
}
template <typename TIN>
__global__ __launch_bounds__(256) void append_bf16_v3_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= a.n) return;
  int b, pos;
  if (a.seq_idx) {
    b = a.seq_idx[i];
    pos = a.pos[i];
  } else {
    b = i / a.L;
    pos = a.start_pos + i % a.L;
  }
  if (b < 0 || b >= a.n_seqs) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_SEQ);
    return;
  }
  const int pidx = pos >= 0 ? pos / a.page_size : -1;
  if (pidx < 0 || pidx >= a.max_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_POS);
    return;
  }
  const int page = a.block_table[(int64_t)b * a.max_pages + pidx];
  if (page < 0 || (int64_t)page >= a.num_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_PAGE);
    return;
  }
  bf16* dst = (bf16*)a.pool + ((int64_t)page * a.page_size + pos % a.page_size) * 576;
  const int64_t ci = (int64_t)i * a.ld_ckv + 8 * lane, ki = (int64_t)i * a.ld_kr;
  // RMSNorm of the latent (the projection, or the sum of its partial products)
  float y[8];
  load8<TIN>(a.ckv, ci, y);
  const int np = n_parts(a, i, 8 * lane);
  for (int q = 1; q < np; ++q) {
    float z[8];
    load8<TIN>(a.ckv, ci + q * a.part_stride, z);
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] += z[k];
  }
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += y[k] * y[k];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / 512.f + a.eps);
  const u32x4 g = *reinterpret_cast<const u32x4*>((const bf16*)a.g_kv + 8 * lane);
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    o[k] = pack_bf16x2(y[2 * k] * inv * bf16_lo(g[k]), y[2 * k + 1] * inv * bf16_hi(g[k]));
  *reinterpret_cast<u32x4*>(dst + 8 * lane) = o;
  // RoPE of the shared decoupled key
  if (lane < 32) {
    const int p = lane;
    float c, s;
    if (a.rope_cs) {
      const float* cs = a.rope_cs + ((int64_t)(i % a.L) * 32 + p) * 2;
      c = cs[0];
      s = cs[1];
    } else {
      rope_cos_sin(pos, p, 64, a.rope, c, s);
    }
    float x0, x1;
    if constexpr (sizeof(TIN) == 4) {
      const float2 v = *reinterpret_cast<const float2*>((const float*)a.kr + ki + 2 * p);
      x0 = v.x;
      x1 = v.y;
      const int npr = n_parts(a, i, 512 + 2 * p);
      for (int q = 1; q < npr; ++q) {
        const float2 w = *reinterpret_cast<const float2*>((const float*)a.kr + ki + q * a.part_stride + 2 * p);
        x0 += w.x;
        x1 += w.y;
      }
    } else {
      const uint32_t v = *reinterpret_cast<const uint32_t*>((const bf16*)a.kr + ki + 2 * p);
      x0 = bf16_lo(v);
      x1 = bf16_hi(v);
    }
    *reinterpret_cast<uint32_t*>(dst + 512 + 2 * p) = pack_bf16x2(c * x0 - s * x1, s * x0 + c * x1);
  }
}

// FP8 cache rows, 656 bytes: c^KV as 512 E4M3 codes, k^R as 64 bf16, then one
// fp32 scale 2^e per 128-value tile of c^KV (the notes page, section 二(三)
// "FP8训练", quantises activations in 1 x 128 tiles, each with its own scale;
// the power-of-two scale is this library's reading).  e is the
// smallest integer with max |x| <= 448 * 2^e over the tile, and each code is
// x * 2^-e (exact) rounded to the nearest E4M3 value, ties to even.
// One wave per token; lane l holds dims 8l .. 8l+7, in tile l / 16.
constexpr int FP8_ROW = 656, FP8_KR = 512, FP8_SCALE = 640;
template <typename TIN>
__global__ __launch_bounds__(64) void append_fp8_kernel(AppendArgs a) {
  const int i = blockIdx.x;
  const int lane = threadIdx.x;
  int b, pos;
  if (a.seq_idx) {
    b = a.seq_idx[i];
    pos = a.pos[i];
  } else {
    b = i / a.L;
    pos = a.start_pos + i % a.L;
  }
  if (b < 0 || b >= a.n_seqs) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_SEQ);
    return;
  }
  const int pidx = pos >= 0 ? pos / a.page_size : -1;
  if (pidx < 0 || pidx >= a.max_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_POS);
    return;
  }
  const int page = a.block_table[(int64_t)b * a.max_pages + pidx];
  if (page < 0 || (int64_t)page >= a.num_pages) {
    if (lane == 0 && a.err_flags) atomicOr(a.err_flags, FLAG_BAD_PAGE);
    return;
  }
  unsigned char* dst = (unsigned char*)a.pool + ((int64_t)page * a.page_size + pos % a.page_size) * FP8_ROW;
  const int64_t ci = (int64_t)i * a.ld_ckv, ki = (int64_t)i * a.ld_kr;
  const auto in = [&](const void* p, int64_t o, int col) {  // col: column of the projection
    float x = ld_as_f32<TIN>(p, o);
    const int np = n_parts(a, i, col);
    for (int q = 1; q < np; ++q) x += ld_as_f32<TIN>(p, o + q * a.part_stride);
    return x;
  };
  // RMSNorm of the latent (d_c = 512)
  float y[8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = in(a.ckv, ci + 8 * lane + k, 8 * lane + k);
    ss += y[k] * y[k];
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / 512.f + a.eps);
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = y[k] * inv * ld_as_f32<bf16>(a.g_kv, 8 * lane + k);
    amax = fmaxf(amax, fabsf(y[k]));
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  // amax = m 2^x, m in [0.5, 1), and 448 = 0.875 * 2^9
  int x2;
  const float m = frexpf(amax, &x2);
  const int e = amax > 0.f ? (m <= 0.875f ? x2 - 9 : x2 - 8) : 0;
  const float down = ldexpf(1.f, -e);
  uint32_t w[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h] * down, y[4 * h + 1] * down, 0, false);
    w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2] * down, y[4 * h + 3] * down, (int)v, true);
  }
  *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(w[0], w[1]);
  if ((lane & 15) == 0) *reinterpret_cast<float*>(dst + FP8_SCALE + 4 * (lane >> 4)) = ldexpf(1.f, e);
  // RoPE of the shared decoupled key (d_rope = 64), bf16
  if (lane < 32) {
    const int p = lane;
    float c, s;
    if (a.rope_cs) {
      const float* cs = a.rope_cs + ((int64_t)(i % a.L) * 32 + p) * 2;
      c = cs[0];
      s = cs[1];
    } else {
      rope_cos_sin(pos, p, 64, a.rope, c, s);
    }
    const float x0 = in(a.kr, ki + 2 * p, 512 + 2 * p), x1 = in(a.kr, ki + 2 * p + 1, 513 + 2 * p);
    *reinterpret_cast<uint32_t*>(dst + FP8_KR + 4 * p) = pack_bf16x2(c * x0 - s * x1, s * x0 + c * x1);
  }
}

__global__ void rope_table_kernel(float* out, int L, int start_pos, int d_rope, RopeParams rp) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = d_rope / 2;
  if (idx >= (int64_t)L * half) return;
  const int t = (int)(idx / half), p = (int)(idx % half);
  float c, s;
  rope_cos_sin(start_pos + t, p, d_rope, rp, c, s);
  out[idx * 2] = c;
  out[idx * 2 + 1] = s;
}

// One wave per row.
template <typename TOUT>
__global__ __launch_bounds__(64) void rmsnorm_kernel(const float* x, int64_t ldx, const void* g, TOUT* out,
                                                     int64_t ldo, int width, float eps) {
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const float* xr = x + r * ldx;
  float ss = 0.f;
  for (int d = lane; d < width; d += 64) ss += xr[d] * xr[d];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)width + eps);
  for (int d = lane; d < width; d += 64) out[r * ldo + d] = from_f32<TOUT>(xr[d] * inv * to_f32(((const TOUT*)g)[d]));
}

// The same for bf16 output and width a multiple of 256 (at most 2048): each
// lane moves 4 consecutive values per access (16-byte loads of x, 8-byte
// loads of g and stores), so a wave's access covers 1 KB of the row.
constexpr int RMS4_MAX = 8;  // float4 groups per lane
__global__ __launch_bounds__(64) void rmsnorm4_bf16_kernel(const float* x, int64_t ldx, const bf16* g, bf16* out,
                                                           int64_t ldo, int width, float eps) {
  const int64_t r = blockIdx.x;
  const int lane = threadIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + r * ldx);
  const int nv = width / 256;
  float4 v[RMS4_MAX];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < RMS4_MAX; ++k) {
    if (k < nv) {
      v[k] = xr[lane + 64 * k];
      ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)width + eps);
#pragma unroll
  for (int k = 0; k < RMS4_MAX; ++k) {
    if (k < nv) {
      const int d = 4 * (lane + 64 * k);
      const uint2 gw = *reinterpret_cast<const uint2*>(g + d);
      const float g0 = __uint_as_float(gw.x << 16), g1 = __uint_as_float(gw.x & 0xffff0000u);
      const float g2 = __uint_as_float(gw.y << 16), g3 = __uint_as_float(gw.y & 0xffff0000u);
      *reinterpret_cast<uint2*>(out + r * ldo + d) =
          make_uint2(pack_bf16x2(v[k].x * inv * g0, v[k].y * inv * g1), pack_bf16x2(v[k].z * inv * g2, v[k].w * inv * g3));
    }
  }
}

// One thread per rotated pair.
template <typename TOUT>
__global__ void rope_heads_kernel(const float* x, const float* cs, int table_rows, TOUT* out, int64_t ld_out,
                                  int out_off, int64_t T, int H, int d_rope) {
  const int half = d_rope / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * H * half) return;
  const int p = (int)(idx % half);
  const int64_t th = idx / half;  // t * H + h
  const int64_t t = th / H;
  const float* c = cs + ((t % table_rows) * half + p) * 2;
  const float x0 = x[th * d_rope + 2 * p], x1 = x[th * d_rope + 2 * p + 1];
  TOUT* o = out + th * ld_out + out_off;
  o[2 * p] = from_f32<TOUT>(c[0] * x0 - c[1] * x1);
  o[2 * p + 1] = from_f32<TOUT>(c[1] * x0 + c[0] * x1);
}

unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  dim3 grid((unsigned)a.n), block(64);
  if (a.fp8_cache) {  // bf16 compute, d_c = 512, d_rope = 64 (checked by the caller)
    if (a.in_f32)
      hipLaunchKernelGGL((append_fp8_kernel<float>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((append_fp8_kernel<bf16>), grid, block, 0, st, a);
  } else if (a.bf16_cache && a.d_c == 512 && a.d_rope == 64) {
    const dim3 g4((unsigned)((a.n + 3) / 4)), b4(256);
    if (a.in_f32)
      hipLaunchKernelGGL((append_bf16_v3_kernel<float>), g4, b4, 0, st, a);
    else
      hipLaunchKernelGGL((append_bf16_v3_kernel<bf16>), g4, b4, 0, st, a);
  } else if (a.bf16_cache) {
    if (a.in_f32)
      hipLaunchKernelGGL((append_kernel<float, bf16>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((append_kernel<bf16, bf16>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((append_kernel<float, float>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_rope_table(float* out, int32_t L, int32_t start_pos, int32_t d_rope, const RopeParams& rp,
                             hipStream_t st) {
  const int64_t n = (int64_t)L * (d_rope / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, out, L, start_pos, d_rope, rp);
  return hipGetLastError();
}

namespace {
template <typename TOUT>
__global__ void sum_partials_kernel(const float* p, int S, int64_t n4, TOUT* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  float4 acc = reinterpret_cast<const float4*>(p)[i];
  for (int z = 1; z < S; ++z) {
    const float4 v = reinterpret_cast<const float4*>(p)[(int64_t)z * n4 + i];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  out[4 * i] = from_f32<TOUT>(acc.x);
  out[4 * i + 1] = from_f32<TOUT>(acc.y);
  out[4 * i + 2] = from_f32<TOUT>(acc.z);
  out[4 * i + 3] = from_f32<TOUT>(acc.w);
}
}  // namespace

hipError_t launch_sum_partials(const float* p, int32_t S, int64_t n, void* out, int32_t bf16_out, hipStream_t st) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  if (bf16_out)
    hipLaunchKernelGGL((sum_partials_kernel<bf16>), dim3(blocks_for(n4, 256)), dim3(256), 0, st, p, S, n4, (bf16*)out);
  else
    hipLaunchKernelGGL((sum_partials_kernel<float>), dim3(blocks_for(n4, 256)), dim3(256), 0, st, p, S, n4,
                       (float*)out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int64_t ldx, const void* g, void* out, int64_t ldo, int32_t rows,
                          int32_t width, float eps, int32_t bf16_io, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
  if (bf16_io && width % 256 == 0 && width <= 256 * RMS4_MAX && ldx % 4 == 0 && ldo % 4 == 0 && al(x, 16) &&
      al(out, 8) && al(g, 8))
    hipLaunchKernelGGL(rmsnorm4_bf16_kernel, dim3(rows), dim3(64), 0, st, x, ldx, (const bf16*)g, (bf16*)out, ldo,
                       width, eps);
  else if (bf16_io)
    hipLaunchKernelGGL((rmsnorm_kernel<bf16>), dim3(rows), dim3(64), 0, st, x, ldx, g, (bf16*)out, ldo, width, eps);
  else
    hipLaunchKernelGGL((rmsnorm_kernel<float>), dim3(rows), dim3(64), 0, st, x, ldx, g, (float*)out, ldo, width, eps);
  return hipGetLastError();
}

hipError_t launch_rope_heads(const float* x, const float* cs, int32_t table_rows, void* out, int64_t ld_out,
                             int32_t out_off, int32_t T, int32_t H, int32_t d_rope, int32_t bf16_out, hipStream_t st) {
  const int64_t n = (int64_t)T * H * (d_rope / 2);
  if (n <= 0) return hipSuccess;
  if (bf16_out)
    hipLaunchKernelGGL((rope_heads_kernel<bf16>), dim3(blocks_for(n, 256)), dim3(256), 0, st, x, cs, table_rows,
                       (bf16*)out, ld_out, out_off, (int64_t)T, H, d_rope);
  else
    hipLaunchKernelGGL((rope_heads_kernel<float>), dim3(blocks_for(n, 256)), dim3(256), 0, st, x, cs, table_rows,
                       (float*)out, ld_out, out_off, (int64_t)T, H, d_rope);
  return hipGetLastError();
}

}  // namespace mla
