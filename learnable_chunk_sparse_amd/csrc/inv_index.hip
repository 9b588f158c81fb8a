// Inverse index of a top-K selection: for every (batch, KV head) and chunk c,
// the list of (position, slot) pairs whose selection holds c, in ascending
// position order. The chunk-major forward walks these lists (each selected
// chunk is loaded once for all the rows that chose it) and the backward's
// key-block pass reads them to find each key block's chunk rows.
//
// A counting sort per (b, KV head) whose order is fixed by the data alone, so
// that every run lists the same entries in the same places (the backward's
// sums over a chunk's rows then run in one order):
//   hist        positions are cut into ns ranges; each range counts its
//               selections per chunk in LDS        -> cnt[bg][range][c]
//   range scan  per chunk, exclusive scan over the ranges (in place) and the
//               chunk's total                      -> off[bg][c] = total
//   chunk scan  exclusive scan of the totals       -> off[bg][c] = first slot,
//                                                     off[bg][C] = entries
//   fill        each range walks its positions in order, a few positions at a
//               time; an entry's rank among the step's entries of the same
//               chunk comes from an LDS bit mask (bit = position in the step,
//               set with an order-free atomic OR), so its slot is the chunk's
//               cursor plus the number of same-chunk bits below its own.
// Entry format: (position << 6) | slot. Optionally rank[bg][position][slot]
// records the entry's index in the list (position-major, for readers that go
// from a selection to its entry).
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>

namespace hils {

namespace {

__global__ __launch_bounds__(256) void k_ix_hist(const int32_t* __restrict__ topk_idx,
                                                 int* __restrict__ cnt, int N, int K, int C, int ns) {
  extern __shared__ int hist[];
  const int sp = blockIdx.x, bg = blockIdx.y, tid = threadIdx.x;
  for (int c = tid; c < C; c += 256) hist[c] = 0;
  __syncthreads();
  const long per = ((long)N + ns - 1) / ns;
  const long i0 = sp * per, i1 = min((long)N, i0 + per);
  const int32_t* src = topk_idx + (long)bg * N * K;
  long x = i0 * K + tid;
  if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0) {
    // 16-byte loads, four per thread in flight (the range starts and ends on
    // a multiple of K, so on whole vectors)
    const int4* s4 = reinterpret_cast<const int4*>(src + i0 * K);
    const long n4 = (i1 - i0) * K / 4;
    for (long v = tid; v < n4; v += 4 * 256) {
      int4 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = v + 256 * u < n4 ? s4[v + 256 * u] : int4{-1, -1, -1, -1};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cs[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (cs[j] >= 0 && cs[j] < C) atomicAdd(&hist[cs[j]], 1);
      }
    }
    x = i1 * K;  // done
  }
  for (; x < i1 * K; x += 256) {
    const int c = src[x];
    if (c >= 0 && c < C) atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  int* dst = cnt + ((long)bg * ns + sp) * C;
  for (int c = tid; c < C; c += 256) dst[c] = hist[c];
}

// one thread per chunk: exclusive scan over the ranges in place, total to off
__global__ __launch_bounds__(256) void k_ix_range_scan(int* __restrict__ cnt, int* __restrict__ off,
                                                       int C, int ns) {
  const int c = blockIdx.x * 256 + threadIdx.x, bg = blockIdx.y;
  if (c >= C) return;
  int* col = cnt + (long)bg * ns * C + c;
  int s = 0;
  int r = 0;
  // eight ranges' counts loaded together, then scanned in order
  for (; r + 8 <= ns; r += 8) {
    int x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = col[(long)(r + j) * C];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      col[(long)(r + j) * C] = s;
      s += x[j];
    }
  }
  for (; r < ns; ++r) {
    const int x = col[(long)r * C];
    col[(long)r * C] = s;
    s += x;
  }
  off[(long)bg * (C + 1) + c] = s;
}

// one workgroup per (b, KV head): exclusive scan of the chunk totals
__global__ __launch_bounds__(256) void k_ix_chunk_scan(int* __restrict__ off, int C) {
  __shared__ int wsum[4];
  int* a = off + (long)blockIdx.x * (C + 1);
  const int tot = block_excl_scan(a, C, wsum);
  if (threadIdx.x == 0) a[C] = tot;
}

// Ranges walk their positions SB at a time (SB K <= 512 entries, two per
// thread, SB <= 32 bits of the masks); the next step's ids are loaded while
// the current step is placed.
__global__ __launch_bounds__(256) void k_ix_fill(const int32_t* __restrict__ topk_idx,
                                                 const int* __restrict__ cnt, const int* __restrict__ off,
                                                 int* __restrict__ lst, int* __restrict__ rank, int N,
                                                 int K, int C, int ns) {
  extern __shared__ int smem[];
  int* cur = smem;                                           // [C] next slot of each chunk
  unsigned* msk = reinterpret_cast<unsigned*>(smem + C);     // [C] chunk's positions in the step
  const int sp = blockIdx.x, bg = blockIdx.y, tid = threadIdx.x;
  const int* cb = cnt + ((long)bg * ns + sp) * C;
  const int* ob = off + (long)bg * (C + 1);
  for (int c = tid; c < C; c += 256) {
    cur[c] = ob[c] + cb[c];
    msk[c] = 0u;
  }
  __syncthreads();
  const long per = ((long)N + ns - 1) / ns;
  const long i0 = sp * per, i1 = min((long)N, i0 + per);
  const int32_t* src = topk_idx + (long)bg * N * K;
  int* dst = lst + (long)bg * N * K;
  const int SB = min(32, 512 / K);
  int pl[2], kk[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    pl[u] = (tid + 256 * u) / K;
    kk[u] = tid + 256 * u - pl[u] * K;
  }
  auto fetch = [&](long i, int u) __attribute__((always_inline)) {
    const long pos = i + pl[u];
    int c = -1;
    if (pl[u] < SB && pos < i1) c = src[pos * K + kk[u]];
    return c < C ? c : -1;
  };
  int cn[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) cn[u] = fetch(i0, u);
  for (long i = i0; i < i1; i += SB) {
    int c[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      c[u] = cn[u];
      cn[u] = i + SB < i1 ? fetch(i + SB, u) : -1;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (c[u] >= 0) atomicOr(&msk[c[u]], 1u << pl[u]);
    __syncthreads();
    unsigned m[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      m[u] = 0u;
      if (c[u] >= 0) {
        m[u] = msk[c[u]];
        const long pos = i + pl[u];
        const int e = cur[c[u]] + __popc(m[u] & ((1u << pl[u]) - 1u));
        dst[e] = (int)((pos << 6) | kk[u]);
        if (rank != nullptr) rank[((size_t)bg * N + pos) * K + kk[u]] = e;
      }
    }
    __syncthreads();
    // the step's last position holding c advances the cursor and clears the mask
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (c[u] >= 0 && (m[u] >> pl[u]) == 1u) {
        cur[c[u]] += __popc(m[u]);
        msk[c[u]] = 0u;
      }
    __syncthreads();
  }
}

}  // namespace

// position ranges: enough workgroups to fill the chip, at least 256 positions each
int inv_ranges(const Dims& p) {
  const long bg = (long)p.B * p.Hkv;
  long ns = (2048 + bg - 1) / bg;
  ns = std::min<long>(ns, (p.N + 255) / 256);
  return (int)std::max<long>(ns, 1);
}

bool inv_index_ok(const Dims& p) {
  // the fill keeps a cursor and a mask per chunk in LDS; entries hold the
  // position above a 6-bit slot in an int
  return p.C <= INV_MAX_CHUNKS && (long)p.N * 64 < (1L << 31) && p.K <= 32;
}

size_t inv_index_carve(const Dims& p, void* base, InvIndex* out, bool with_rank) {
  char* c = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + o : nullptr;
    o += (bytes + 255) & ~(size_t)255;
    return ptr;
  };
  const size_t bg = (size_t)p.B * p.Hkv;
  out->ns = inv_ranges(p);
  out->cnt = (int*)take(bg * out->ns * (size_t)p.C * sizeof(int));
  out->off = (int*)take(bg * ((size_t)p.C + 1) * sizeof(int));
  out->lst = (int*)take(bg * (size_t)p.N * p.K * sizeof(int));
  out->rank = with_rank ? (int*)take(bg * (size_t)p.N * p.K * sizeof(int)) : nullptr;
  return o;
}

hipError_t launch_inv_index(const Dims& p, const int32_t* topk_idx, const InvIndex& ix,
                            hipStream_t st) {
  const unsigned bg = (unsigned)(p.B * p.Hkv);
  if (p.C == 0) {
    // no chunk: every list is empty (the scan of no totals writes off[bg][0] = 0)
    hipLaunchKernelGGL(k_ix_chunk_scan, dim3(bg), dim3(256), 0, st, ix.off, 0);
    return hipGetLastError();
  }
  const size_t hl = (size_t)p.C * sizeof(int);
  hipError_t err = hipFuncSetAttribute((const void*)k_ix_hist, hipFuncAttributeMaxDynamicSharedMemorySize, (int)hl);
  if (err != hipSuccess) return err;
  err = hipFuncSetAttribute((const void*)k_ix_fill, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(2 * hl));
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_ix_hist, dim3(ix.ns, bg), dim3(256), hl, st, topk_idx, ix.cnt, p.N, p.K, p.C,
                     ix.ns);
  hipLaunchKernelGGL(k_ix_range_scan, dim3((p.C + 255) / 256, bg), dim3(256), 0, st, ix.cnt, ix.off,
                     p.C, ix.ns);
  hipLaunchKernelGGL(k_ix_chunk_scan, dim3(bg), dim3(256), 0, st, ix.off, p.C);
  hipLaunchKernelGGL(k_ix_fill, dim3(ix.ns, bg), dim3(256), 2 * hl, st, topk_idx, ix.cnt, ix.off,
                     ix.lst, ix.rank, p.N, p.K, p.C, ix.ns);
  return hipGetLastError();
}

}  // namespace hils
