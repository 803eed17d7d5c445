// Device-side work plan of the latent attention (see mla_kernels.h for the
// plan layout): token-balanced chunks of every query row's visible keys and
// the per-workgroup item table, built by one workgroup of 256 threads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"
#include "mla_kernels.h"

namespace mla {

// kv_len of sequence b and whether it is within [s_q, max_kv]
__device__ __forceinline__ int kv_len_of(const AttnArgs& a, int b, bool& ok) {
  const int kv = a.kv_lens ? a.kv_lens[b] : a.uniform_kv;
  ok = kv >= a.s_q && kv <= a.max_kv;
  return kv;
}

// The whole plan, computed by the 256 threads of the calling workgroup (every
// thread must call it; it synchronises the workgroup).
__device__ inline void plan_body(const AttnArgs& a, int32_t* plan, int32_t target_items, int32_t min_chunk,
                                 int32_t max_chunk) {
  __shared__ long long red_tot[4];
  __shared__ int red_max[4], wsum[4];
  __shared__ int chunk_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n_rows = a.B * a.s_q;
  auto vis = [&](int r, bool report) -> int {  // visible keys of query row r
    const int b = r / a.s_q, s = r % a.s_q;
    bool ok;
    const int kv = kv_len_of(a, b, ok);
    if (!ok) {
      if (report && s == 0 && a.err_flags) atomicOr(a.err_flags, MLA_FLAG_BAD_LEN);
      return 0;
    }
    return kv - a.s_q + s + 1;
  };
  long long tot = 0;
  int mx = 0;
  for (int r = tid; r < n_rows; r += 256) {
    const int v = vis(r, true);
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
    const long long T = red_tot[0] + red_tot[1] + red_tot[2] + red_tot[3];
    const int M = max(max(red_max[0], red_max[1]), max(red_max[2], red_max[3]));
    int chunk = max_chunk;
    if (target_items > 0 && T > 0) {
      // ragged batches get four times as many, smaller, chunks to even out;
      // never more than the item slots the caller provided (max_items, of
      // which 7 stay free for the XCD runs below) can hold: with chunks of at
      // least T / tgt keys a row of v keys takes at most v / chunk + 1 items
      long long tgt = (T * 4 >= 3LL * n_rows * M) ? target_items : 4LL * target_items;
      const long long room = (long long)a.max_items - 7 - n_rows;
      tgt = max(1LL, min(tgt, room));
      const long long c = (T + tgt - 1) / tgt;
      chunk = (int)min<long long>(max_chunk, max<long long>(min_chunk, (c + 31) / 32 * 32));
    }
    plan[1] = chunk;
    chunk_s = chunk;
  }
  __syncthreads();
  const int chunk = chunk_s;
  // exclusive scan of the per-row chunk counts (first item of each row)
  int carry = 0;
  for (int base = 0; base < n_rows; base += 256) {
    const int r = base + tid;
    const int c = r < n_rows ? (vis(r, false) + chunk - 1) / chunk : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = carry;
    for (int w2 = 0; w2 < wv; ++w2) before += wsum[w2];
    if (r < n_rows) plan[2 + r] = before + incl - c;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (tid == 0) {
    plan[2 + n_rows] = carry;
    plan[0] = carry;
  }
  // Per-workgroup item table in launch order (each thread re-reads only the
  // row offsets it wrote itself).  Workgroup i runs on XCD i % 8.  Without
  // longest_first the items go to the XCDs in 8 runs of consecutive launch
  // ordinals, so the chunks of one row (which read the same queries) share an
  // L2; with longest_first the items run in reverse plan order.  The grid has
  // at least n_items + 7 slots.
  // Launch ordinals: the plan order, except that with a few query rows per
  // sequence (s_q <= MAX_COSCHED) chunk i of every row of a sequence are
  // neighbours: they read the same cache pages, so running them at the same
  // time on one XCD lets the L2 serve the second read of each tile.
  constexpr int MAX_COSCHED = 8;
  const int n_items = carry;
  const int per = (n_items + 7) / 8;
  const bool cosched = !a.longest_first && a.s_q > 1 && a.s_q <= MAX_COSCHED;
  int4* info = reinterpret_cast<int4*>(plan + plan_info_offset(n_rows));
  for (int r = tid; r < n_rows; r += 256) {
    const int v = vis(r, false);
    const int c = (v + chunk - 1) / chunk;
    const int first = plan[2 + r];
    int cs[MAX_COSCHED];
    int seq_first = first;  // the sequence's first item (its rows' items are contiguous)
    const int s = r % a.s_q, rb = r - s;
    if (cosched) {
#pragma unroll
      for (int s2 = 0; s2 < MAX_COSCHED; ++s2) {
        cs[s2] = s2 < a.s_q ? (vis(rb + s2, false) + chunk - 1) / chunk : 0;
        if (s2 < s) seq_first -= cs[s2];
      }
    }
    for (int i = 0; i < c; ++i) {
      const int item = first + i;
      int ord = item;
      if (cosched) {  // items of the sequence with a lower chunk index, then this chunk's earlier rows
        ord = seq_first;
#pragma unroll
        for (int s2 = 0; s2 < MAX_COSCHED; ++s2) ord += min(cs[s2], i) + (s2 < s && cs[s2] > i ? 1 : 0);
      }
      const int slot = a.longest_first ? n_items - 1 - item : (ord % per) * 8 + ord / per;
      info[slot] = make_int4(r, i * chunk, min((i + 1) * chunk, v), (item << 1) | (c > 1 ? 1 : 0));
    }
  }
  for (int s3 = tid; s3 < a.max_items; s3 += 256) {
    const bool used = a.longest_first ? s3 < n_items : (s3 / 8 < per && (s3 % 8) * per + s3 / 8 < n_items);
    if (!used) info[s3] = make_int4(0, 0, 0, 0);
  }
}

}  // namespace mla
