// HiLS decode step: one new query per sequence (paper Fig. 6 decode latency;
// nestfrontier "The routing problem": score the chunk summaries, keep the top
// K distant chunks, attend inside them and in the local window).
//
// The step is bound by HBM bandwidth: every distant landmark key is read once
// (the O(L/S) per-token retrieval term), then only the K selected chunks and
// the window. Four launches:
//   k_dec_scan    streaming landmark scan: each wave scores 512 chunks of
//                 one (sequence, KV head) with 16x16x32 MFMAs (rows = the
//                 group's query heads, hi and lo halves of an fp32 query;
//                 columns = chunks), a ring of four 16-chunk steps in flight;
//                 the max over heads is in-lane. The wave then keeps the top
//                 min(K, 512) of its 512 scores (by score, then lower index;
//                 the K-th key found bit by bit from ballots) as candidates, in chunk
//                 order: every chunk of the overall top-K is among them.
//   k_dec_select_window
//                 blocks 0 .. B Hkv - 1: the top-K of one (sequence, KV head)'s
//                 candidates, ties resolved by lower chunk index, the chosen
//                 ids in ascending order (no sort): one wave of ballots for
//                 up to 512 candidates, longer lists by a 4-pass 8-bit radix
//                 select over order-preserving integer keys held in
//                 registers, placed by a prefix sum. The other blocks
//                 run the window units, which do not depend on the selection
//                 and keep HBM busy meanwhile.
//   k_dec_chunks  the selected-chunk units.
//                 A unit is one wave over 64 tokens for all G heads: S^T = K Q^T
//                 on MFMA, softmax, O^T = V^T P^T; the V^T operands come from
//                 the row-major V fragments by a product with the identity
//                 (exact), so nothing is staged in LDS. A chunk unit leaves
//                 (log-weight s_c, weight 1, O_c); a window block leaves its
//                 (max, sum, unnormalised output).
//   k_dec_combine per (sequence, query head): log-sum-exp merge of all units,
//                 which is exactly the fusion softmax over {s_c} and lse_W.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>

namespace hils {

namespace {

constexpr int CPW = 2048;  // chunks per scan workgroup

__device__ __forceinline__ int seq_n(const int32_t* seq_len, int b, int N) {
  if (seq_len == nullptr) return N;
  int n = seq_len[b];
  return n < 1 ? 1 : (n > N ? N : n);
}

// monotone map of a float to uint32 (larger float -> larger key)
__device__ __forceinline__ uint32_t ord_f(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace

// ---------------------------------------------------------------- wave top-K
// exclusive prefix sum over the 64 lanes of a wave; total as well
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  total = __shfl(x, 63, 64);
  return x - v;
}

// The kc = min(Kc, #entries) best entries of a list of at most 512 (score,
// chunk id) entries by (score desc, list position asc), written in list
// order to os / oi (os may be null); slots kc .. Kc-1 get id -1. Entry i
// exists when i < nv and, given an id list, ids[i] >= 0; without one its id
// is c0 + i. Both arrays must hold 512 readable entries. One wave; lane l
// holds entries 8l .. 8l + 7 as order-preserving keys (0 = no entry); the
// exact key T of the kc-th best is found bit by bit from the top with
// wave-wide counts (popcounts of ballots), and the first krem keys equal to
// T (earliest in the list) are taken. Lists in ascending chunk order
// therefore break ties by lower chunk index, and the best Kc of a
// concatenation of such lists are among the lists' own best Kc.
__device__ __forceinline__ void wave_topk(const float* __restrict__ sc, const int32_t* __restrict__ ids,
                                          int c0, int nv, int Kc, float* __restrict__ os,
                                          int32_t* __restrict__ oi) {
  const int lane = threadIdx.x & 63;
  uint32_t kk[8];
  float sv[8];
  int iv[8];
  {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(sc + 8 * lane);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(sc + 8 * lane + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = x0[i];
      sv[4 + i] = x1[i];
    }
    if (ids != nullptr) {
      const int4 y0 = *reinterpret_cast<const int4*>(ids + 8 * lane);
      const int4 y1 = *reinterpret_cast<const int4*>(ids + 8 * lane + 4);
      iv[0] = y0.x; iv[1] = y0.y; iv[2] = y0.z; iv[3] = y0.w;
      iv[4] = y1.x; iv[5] = y1.y; iv[6] = y1.z; iv[7] = y1.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) iv[i] = c0 + 8 * lane + i;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) kk[i] = (8 * lane + i < nv && iv[i] >= 0) ? ord_f(sv[i]) : 0u;
  }
  int nvalid = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) nvalid += __popcll(__ballot(kk[i] != 0u));
  const int kc = min(Kc, nvalid);
  const bool all = nvalid <= kc;
  uint32_t prefix = 0u;
  int krem = kc;
  if (!all) {
    // the kc-th largest key T, bit by bit from the top: the largest T with
    // #(keys >= T) >= kc, each count a popcount of ballots (no LDS, no
    // atomics); krem = how many keys equal to T complete the kc
#pragma unroll 4
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = prefix | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) c += __popcll(__ballot(kk[i] >= t));
      if (c >= kc) prefix = t;
    }
    int above = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) above += __popcll(__ballot(kk[i] > prefix));
    krem = kc - above;
  }
  const uint32_t T = prefix;
  int ties = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ties += (!all && kk[i] == T) ? 1 : 0;
  int tot;
  const int tie0 = wave_excl_scan(ties, tot);
  auto taken = [&](int i, int& tr) __attribute__((always_inline)) {
    const bool eq = !all && kk[i] == T;
    const bool tk = kk[i] != 0u && (all || kk[i] > T || (eq && tr < krem));
    tr += eq ? 1 : 0;
    return tk;
  };
  int cnt = 0;
  {
    int tr = tie0;
#pragma unroll
    for (int i = 0; i < 8; ++i) cnt += taken(i, tr) ? 1 : 0;
  }
  int o = wave_excl_scan(cnt, tot);
  {
    int tr = tie0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (taken(i, tr)) {
        if (os != nullptr) os[o] = sv[i];
        oi[o] = iv[i];
        ++o;
      }
    }
  }
  for (int x = tot + lane; x < Kc; x += 64) {
    if (os != nullptr) os[x] = 0.f;
    oi[x] = -1;
  }
}

// ---------------------------------------------------------------- scan
// D[head][chunk] = q_h . kL_c: the query heads are the A operand (rows; hi
// and lo bf16 halves of an fp32 query accumulate into the same product), the
// landmark rows the B operand (columns), so lane (g, c) ends with the scores
// of chunk c for heads 4 g .. 4 g + 3 and the max over heads is in-lane.
// Paged caches (PG): pages of 64 tokens, k / v [P, Hkv, 64, d], landmark rows
// [P, Hkv, d] and biases [P, Hkv]; ptab [B, maxp] holds the page of chunk c
// of sequence b (a chunk is a page).
template <typename T, typename QT, int G, int DH, bool PG>
__global__ __launch_bounds__(256) void k_dec_scan(const QT* __restrict__ qs, const T* __restrict__ kL,
                                                  const T* __restrict__ e,
                                                  const int32_t* __restrict__ seq_len,
                                                  const int32_t* __restrict__ ptab, int maxp,
                                                  float* __restrict__ cand_s, int32_t* __restrict__ cand_i,
                                                  int cstride, int Kc, int N, int C, int Hkv, int W,
                                                  int S, float scale) {
  typedef typename Frag<T>::type FT;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  constexpr int KS = DH / 32;
  constexpr int NST = CPW / 64;  // 16-chunk steps per wave
  constexpr int PD = 4;          // steps in flight per wave
  static_assert(G <= 8 && NST % PD == 0 && CPW / 4 == 512, "scan shape");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int gl = lane >> 4, col = lane & 15;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int n = seq_n(seq_len, b, N);
  const int nd = n_distant(n - 1, W, S);
  const int c_w = split * CPW + (CPW / 4) * w;  // this wave's first chunk
  if (c_w >= nd) return;
  // landmark row of chunk c: bg C + c, or (page of c) Hkv + g; a paged
  // wave first copies the page ids of its chunks into LDS
  __shared__ int spg[PG ? 4 : 1][PG ? CPW / 4 : 1];
  if constexpr (PG) {
#pragma unroll
    for (int x = lane; x < CPW / 4; x += 64) spg[w][x] = ptab[(size_t)b * maxp + min(c_w + x, nd - 1)];
    wave_lds_sync();
  }
  auto lrow = [&](int c) __attribute__((always_inline)) {
    if constexpr (PG) return (size_t)spg[w][c - c_w] * Hkv + g;
    else return (size_t)bg * C + c;
  };
  // ring of PD steps: landmark rows chunk c_w + 16 st + col, dims 8 gl + 32 ks
  // (B operand), and the chunk's bias
  FT kb[PD][KS];
  float eb[PD];
  // waves walk their steps from different starting points, so that the
  // thousands of concurrent streams (whose bases are a power of two apart)
  // spread over the HBM channels instead of moving through them in lockstep
  const int rot = (bg * 7 + split * 13 + w * 5) & (NST - 1);
  auto cstep = [&](int st) __attribute__((always_inline)) { return c_w + 16 * ((st + rot) & (NST - 1)); };
  auto load = [&](int st, FT (&kd)[KS], float& ed) __attribute__((always_inline)) {
    const size_t r = lrow(min(cstep(st) + col, nd - 1));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kd[ks] = ld8<T>(kL + r * DH + 8 * gl + 32 * ks);
    ed = to_f<T>(e[r]);
  };
#pragma unroll
  for (int j = 0; j < PD; ++j) load(j, kb[j], eb[j]);
  // A operand: row h < G holds query head h (hi part; lo part in qlo)
  FT qa[KS], qlo[HAS_LO ? KS : 1];
  {
    const bool live = col < G;
    const QT* src = qs + ((size_t)b * Hq + g * G + (live ? col : 0)) * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // one vector load per fragment (no per-element branches: those drain
      // the landmark loads already in flight)
      const auto raw = ld8<QT>(src + 32 * ks);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = live ? (float)raw[j] : 0.f;
      qa[ks] = pack8<T>(x);
      if constexpr (HAS_LO) {
        const u16x8 hb = __builtin_bit_cast(u16x8, qa[ks]);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] -= bf2f(hb[j]);
        qlo[ks] = pack8<T>(x);
      }
    }
  }
  // scores are collected in LDS; the wave then keeps its own top-K as
  // candidates for the selection
  __shared__ __align__(16) float sbuf[4][CPW / 4];
  float* sw = sbuf[w];
  // fully unrolled, so the waits on the ring are exact (a loop back edge
  // would drain every load in flight)
#pragma unroll
  for (int st = 0; st < NST; st += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = mma16(qa[ks], kb[j][ks], acc);
        if constexpr (HAS_LO) acc = mma16(qlo[ks], kb[j][ks], acc);
      }
      float v = acc[0];
#pragma unroll
      for (int i = 1; i < (G < 4 ? G : 4); ++i) v = fmaxf(v, acc[i]);
      if constexpr (G == 8) {  // heads 4..7 sit in the lanes 16 above
        auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float out = fmaf(v, scale, eb[j]);
      if (gl == 0) sw[cstep(st + j) - c_w + col] = out;
      if (st + j + PD < NST) load(st + j + PD, kb[j], eb[j]);
    }
  }
  wave_lds_sync();
  const size_t ob = (size_t)bg * cstride + (size_t)(c_w / (CPW / 4)) * Kc;
  wave_topk(sw, nullptr, c_w, nd - c_w, Kc, cand_s + ob, cand_i + ob);
}

// ---------------------------------------------------------------- select
// exclusive prefix sum of v over the 256 threads of the block; total as well
__device__ __forceinline__ int block_scan256(int v, int* wsum, int& total) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s2 = wsum[j];
    base += j < w ? s2 : 0;
    tot += s2;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// The K best of the candidate list (sc, id)[0..n) of one (sequence, KV head)
// by (score desc, chunk asc), written as ascending chunk ids, -1 padded; one
// 256-thread block. The list is in ascending chunk order (id -1 = no entry),
// so list order breaks ties. Thread t holds the order-preserving integer keys
// of entries [t PER, t PER + PER) in registers (contiguous ranges, so prefix
// sums follow list order); the exact key T of the K-th best comes from a
// 4-pass 8-bit radix select, and the first krem keys equal to T are taken.
template <int PER>
__device__ __forceinline__ void select_block(const float* __restrict__ sc, const int32_t* __restrict__ id,
                                             int n, int K, int32_t* __restrict__ sel,
                                             int32_t* __restrict__ topk_out) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem;
  const int t = threadIdx.x;
  const int lo = t * PER;
  // vector loads (the lists are padded to at least 256 PER entries); key 0
  // marks no entry (no finite score maps to 0)
  uint32_t key[PER];
  int cid[PER];
#pragma unroll
  for (int j4 = 0; j4 < PER / 4; ++j4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(sc + lo + 4 * j4);
    const int4 y = *reinterpret_cast<const int4*>(id + lo + 4 * j4);
    const int yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = lo + 4 * j4 + i < n && yy[i] >= 0;
      key[4 * j4 + i] = ok ? ord_f(x[i]) : 0u;
      cid[4 * j4 + i] = yy[i];
    }
  }
  int nv = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) nv += key[j] != 0u ? 1 : 0;
  int tot;
  nv = block_scan256(nv, wsum, tot);
  const bool take_all = tot <= K;
  if (t == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_krem = K;
  }
  if (!take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[t] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (key[j] != 0u && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255], 1);
      __syncthreads();
      if (t < 64) {
        // lane t holds bins 4t .. 4t+3; keys in higher bins rank above
        int h4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h4[j] = hist[4 * t + j];
          sum += h4[j];
        }
        int x = sum;  // suffix sum over lanes >= t
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_down(x, o, 64);
          if (t + o < 64) x += y;
        }
        const int krem = s_krem;
        int above = x - sum;
        for (int j = 3; j >= 0; --j) {
          const int with = above + h4[j];
          if (above < krem && krem <= with) {
            s_prefix = prefix | ((uint32_t)(4 * t + j) << shift);
            s_mask = mask | (255u << shift);
            s_krem = krem - above;
          }
          above = with;
        }
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const int krem = s_krem;
  int ties = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) ties += (!take_all && key[j] == T) ? 1 : 0;
  const int tie0 = block_scan256(ties, wsum, tot);
  // entry j is taken: above T, or equal to T among the first krem ties (tr
  // counts the ties before it)
  auto taken = [&](int j, int& tr) __attribute__((always_inline)) {
    const bool eq = !take_all && key[j] == T;
    const bool tk = key[j] != 0u && (take_all || key[j] > T || (eq && tr < krem));
    tr += eq ? 1 : 0;
    return tk;
  };
  int cnt = 0;
  {
    int tr = tie0;
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt += taken(j, tr) ? 1 : 0;
  }
  int o = block_scan256(cnt, wsum, tot);
  {
    int tr = tie0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (taken(j, tr)) {
        sel[o] = cid[j];
        if (topk_out != nullptr) topk_out[o] = cid[j];
        ++o;
      }
    }
  }
  for (int k2 = tot + t; k2 < K; k2 += 256) {
    sel[k2] = -1;
    if (topk_out != nullptr) topk_out[k2] = -1;
  }
}

// longer candidate lists: keys re-read on every pass, eight per thread and
// iteration (the lists are padded to a multiple of 8)
__device__ __forceinline__ void select_block_big(const float* __restrict__ sc, const int32_t* __restrict__ id,
                                                 int n, int K, int32_t* __restrict__ sel,
                                                 int32_t* __restrict__ topk_out) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem;
  const int t = threadIdx.x;
  auto keys8 = [&](int c0, uint32_t (&kk)[8], int (&ci)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(sc + c0 + 4 * h);
      const int4 y = *reinterpret_cast<const int4*>(id + c0 + 4 * h);
      const int yy[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = c0 + 4 * h + i < n && yy[i] >= 0;
        kk[4 * h + i] = ok ? ord_f(a[i]) : 0u;
        ci[4 * h + i] = yy[i];
      }
    }
  };
  int nv = 0;
  for (int c0 = 8 * t; c0 < n; c0 += 2048) {
    uint32_t kk[8];
    int ci[8];
    keys8(c0, kk, ci);
#pragma unroll
    for (int i = 0; i < 8; ++i) nv += kk[i] != 0u ? 1 : 0;
  }
  int tot;
  block_scan256(nv, wsum, tot);
  const bool take_all = tot <= K;
  if (t == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_krem = K;
  }
  __syncthreads();
  if (!take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[t] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int c0 = 8 * t; c0 < n; c0 += 2048) {
        uint32_t kk[8];
        int ci[8];
        keys8(c0, kk, ci);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (kk[i] != 0u && (kk[i] & mask) == prefix) atomicAdd(&hist[(kk[i] >> shift) & 255], 1);
      }
      __syncthreads();
      if (t < 64) {
        int h4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h4[j] = hist[4 * t + j];
          sum += h4[j];
        }
        int x = sum;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_down(x, o, 64);
          if (t + o < 64) x += y;
        }
        const int krem = s_krem;
        int above = x - sum;
        for (int j = 3; j >= 0; --j) {
          const int with = above + h4[j];
          if (above < krem && krem <= with) {
            s_prefix = prefix | ((uint32_t)(4 * t + j) << shift);
            s_mask = mask | (255u << shift);
            s_krem = krem - above;
          }
          above = with;
        }
      }
      __syncthreads();
    }
  }
  const uint32_t T = s_prefix;
  const int krem = s_krem;
  // contiguous ranges of a multiple of 8 entries per thread (prefix sums
  // follow list order)
  const int per = ((n + 255) / 256 + 7) / 8 * 8;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  int ties = 0;
  if (!take_all)
    for (int c0 = lo; c0 < hi; c0 += 8) {
      uint32_t kk[8];
      int ci[8];
      keys8(c0, kk, ci);
#pragma unroll
      for (int i = 0; i < 8; ++i) ties += kk[i] == T ? 1 : 0;
    }
  const int tie0 = block_scan256(ties, wsum, tot);
  auto taken = [&](uint32_t key, int& tr) __attribute__((always_inline)) {
    const bool eq = !take_all && key == T;
    const bool tk = key != 0u && (take_all || key > T || (eq && tr < krem));
    tr += eq ? 1 : 0;
    return tk;
  };
  int cnt = 0;
  {
    int tr = tie0;
    for (int c0 = lo; c0 < hi; c0 += 8) {
      uint32_t kk[8];
      int ci[8];
      keys8(c0, kk, ci);
#pragma unroll
      for (int i = 0; i < 8; ++i) cnt += taken(kk[i], tr) ? 1 : 0;
    }
  }
  const int out0 = block_scan256(cnt, wsum, tot);
  {
    int tr = tie0, o = out0;
    for (int c0 = lo; c0 < hi; c0 += 8) {
      uint32_t kk[8];
      int ci[8];
      keys8(c0, kk, ci);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (taken(kk[i], tr)) {
          sel[o] = ci[i];
          if (topk_out != nullptr) topk_out[o] = ci[i];
          ++o;
        }
      }
    }
  }
  for (int k2 = tot + t; k2 < K; k2 += 256) {
    sel[k2] = -1;
    if (topk_out != nullptr) topk_out[k2] = -1;
  }
}

// ---------------------------------------------------------------- attention units
// partials per (bg, unit, head): pml = [m, l], po = U[0..DH)
struct DecArgs {
  const int32_t* seq_len;
  const int32_t* ptab;  // paged caches: page of chunk c of sequence b at b maxp + c
  int maxp;
  const int32_t* sel;
  float *pml, *po;
  int N, C, Hkv, K, W, S, units;
  float scale;
};

// One wave: units u0, u0 + us, ... (up to NUW of them) of (sequence, KV
// head) bg, software-pipelined: the next unit's K rows are requested as soon
// as the current scores are formed, its V rows as soon as the current output
// is, so loads stay in flight while the wave computes.
template <typename T, typename QT, int G, int DH, int NUW, bool PG>
__device__ __forceinline__ void dec_units(const T* __restrict__ q, const QT* __restrict__ qs,
                                          const T* __restrict__ k, const T* __restrict__ v,
                                          const T* __restrict__ kL, const T* __restrict__ e,
                                          const DecArgs& a, int bg, int u0, int us) {
  typedef typename Frag<T>::type FT;
  constexpr int KS = DH / 32, MB = DH / 16;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  const int lane = threadIdx.x & 63;
  const int gl = lane >> 4, col = lane & 15;
  const int N = a.N, C = a.C, Hkv = a.Hkv, K = a.K, S = a.S, units = a.units;
  const float scale = a.scale;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int n = seq_n(a.seq_len, b, N);
  const int ws = n_distant(n - 1, a.W, S) * S;
  // what each unit covers (wave-uniform): a selected chunk, or a window block
  // (both 64-token aligned: one page of a paged cache)
  int uu[NUW], t0[NUW], cnt[NUW], chunk[NUW];
  size_t kvb[NUW], lmr[NUW];  // first K/V row of the unit, landmark row of its chunk
#pragma unroll
  for (int j = 0; j < NUW; ++j) {
    const int u = u0 + j * us;
    uu[j] = u;
    chunk[j] = -1;
    if (u < K) {
      chunk[j] = __builtin_amdgcn_readfirstlane(a.sel[(size_t)bg * K + u]);
      t0[j] = chunk[j] >= 0 ? chunk[j] * S : 0;
      cnt[j] = chunk[j] >= 0 ? S : 0;
    } else {
      t0[j] = ws + 64 * (u - K);
      cnt[j] = u < units ? min(64, n - t0[j]) : 0;
      if (cnt[j] <= 0) t0[j] = 0;
    }
    const int cl = chunk[j] >= 0 ? chunk[j] : 0;
    if constexpr (PG) {
      const size_t pk = (size_t)__builtin_amdgcn_readfirstlane(a.ptab[(size_t)b * a.maxp + t0[j] / 64]);
      const size_t pl = (size_t)__builtin_amdgcn_readfirstlane(a.ptab[(size_t)b * a.maxp + cl]);
      kvb[j] = (pk * Hkv + g) * 64;
      lmr[j] = pl * Hkv + g;
    } else {
      kvb[j] = (size_t)bg * N + t0[j];
      lmr[j] = (size_t)bg * C + cl;
    }
  }
  // loop-invariant operands: raw query heads (B operand of S^T = K Q^T), the
  // calibrated query heads for the landmark score (B operand; hi + lo of an
  // fp32 query), identity fragments I_h[k][c] = (k == 16 h + c)
  FT qf[KS], qsf[KS], qsl[HAS_LO ? KS : 1], idf[2];
  {
    const int h = col < G ? col : 0;
    const T* src = q + ((size_t)b * Hq + g * G + h) * DH + 8 * gl;
    const QT* srs = qs + ((size_t)b * Hq + g * G + h) * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const FT raw = ld8<T>(src + 32 * ks);
      const auto rs = ld8<QT>(srs + 32 * ks);
      float x[8], y[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        x[jj] = col < G ? (float)raw[jj] : 0.f;
        y[jj] = col < G ? (float)rs[jj] : 0.f;
      }
      qf[ks] = pack8<T>(x);
      qsf[ks] = pack8<T>(y);
      if constexpr (HAS_LO) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) y[jj] -= (float)qsf[ks][jj];
        qsl[ks] = pack8<T>(y);
      }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      float x[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = (8 * gl + jj == 16 * hh + col) ? 1.f : 0.f;
      idf[hh] = pack8<T>(x);
    }
  }
  // register sets of one unit: K and V rows (token 16 tb + col, dims 8 gl +
  // 32 ks) and the chunk's landmark row (every A row = kL_c)
  FT kf[4][KS], vf[4][KS], kr[KS];
  auto loadK = [&](int j) __attribute__((always_inline)) {
    const T* kb = k + kvb[j] * DH;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tok = 16 * tb + col < cnt[j] ? 16 * tb + col : 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[tb][ks] = ld8<T>(kb + (size_t)tok * DH + 8 * gl + 32 * ks);
    }
    const T* krow = kL + lmr[j] * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = ld8<T>(krow + 32 * ks);
  };
  auto loadV = [&](int j) __attribute__((always_inline)) {
    const T* vb = v + kvb[j] * DH;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int tok = 16 * tb + col < cnt[j] ? 16 * tb + col : 0;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) vf[tb][ks] = ld8<T>(vb + (size_t)tok * DH + 8 * gl + 32 * ks);
    }
  };
  loadK(0);
  loadV(0);
#pragma unroll
  for (int j = 0; j < NUW; ++j) {
    // scores of the unit's tokens, and (chunk units) the landmark score of
    // every head: D[row][col = h] = kL_c . q_hat_h
    f32x4 sacc[4], lm = zero4();
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      sacc[tb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[tb] = mma16(kf[tb][ks], qf[ks], sacc[tb]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      lm = mma16(kr[ks], qsf[ks], lm);
      if constexpr (HAS_LO) lm = mma16(kr[ks], qsl[ks], lm);
    }
    const int cj = cnt[j], chj = chunk[j];
    const float ebias = chj >= 0 ? to_f<T>(e[lmr[j]]) : 0.f;
    if (j + 1 < NUW) loadK(j + 1);
    float mx = NEG_INF;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int tok = 16 * tb + 4 * gl + ii;
        const float x = tok < cj ? sacc[tb][ii] * scale : NEG_INF;
        sacc[tb][ii] = x;
        mx = fmaxf(mx, x);
      }
    mx = col_max4(mx);
    float ls = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float x = sacc[tb][ii];
        const float p = x == NEG_INF ? 0.f : __expf(x - mx);
        sacc[tb][ii] = p;
        ls += p;
      }
    ls = col_sum4(ls);
    f32x4 oacc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb] = zero4();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // 32-token steps
      const FT pf = pk8<T>(sacc[2 * ks], sacc[2 * ks + 1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // V^T rows 16 mb .. 16 mb + 15 over the step's tokens, in the token
        // order of the P^T fragment
        const int kd = mb >> 1, hs = mb & 1;
        const FT vt = pk8<T>(mma16(vf[2 * ks][kd], idf[hs], zero4()),
                             mma16(vf[2 * ks + 1][kd], idf[hs], zero4()));
        oacc[mb] = mma16(vt, pf, oacc[mb]);
      }
    }
    if (j + 1 < NUW) loadV(j + 1);
    const int u = uu[j];
    if (u < units && col < G) {
      float mval = mx, lval = ls, coef = 1.f;
      if (chj >= 0) {
        // a selected chunk enters the fusion as one term: log-weight s_c,
        // weight 1, vector O_c
        mval = fmaf(lm[0], scale, ebias);
        lval = 1.f;
        coef = 1.f / ls;
      }
      float* pm = a.pml + ((size_t)bg * units + u) * G * 2;
      float* pv = a.po + ((size_t)bg * units + u) * G * DH;
      if (gl == 0) {
        pm[2 * col] = mval;
        pm[2 * col + 1] = lval;
      }
      float* ph = pv + (size_t)col * DH + 4 * gl;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4*>(ph + 16 * mb) = oacc[mb] * coef;
    }
  }
}

// selections (one block per (sequence, KV head)) and, alongside in the same
// launch, the window units, which do not depend on them (bf16: at most 128
// registers with the accumulators, four waves per SIMD)
template <typename T, typename QT, int G, int DH, int PER, bool PG>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? 4 : 1) void k_dec_select_window(const float* __restrict__ cand_s,
                                                           const int32_t* __restrict__ cand_i,
                                                           int32_t* __restrict__ topk_out, int cstride,
                                                           int Kc, int nbg, int wpb, const T* __restrict__ q,
                                                           const QT* __restrict__ qs,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const T* __restrict__ kL,
                                                           const T* __restrict__ e, DecArgs a) {
  const int blk = blockIdx.x;
  if (blk < nbg) {
    const int bg = blk, b = bg / a.Hkv;
    const int nd = n_distant(seq_n(a.seq_len, b, a.N) - 1, a.W, a.S);
    // candidates: Kc per 512 scanned chunks
    const int n = (nd + 511) / 512 * Kc;
    int32_t* sl = const_cast<int32_t*>(a.sel) + (size_t)bg * a.K;
    int32_t* to = topk_out != nullptr ? topk_out + (size_t)bg * a.K : nullptr;
    const float* cs = cand_s + (size_t)bg * cstride;
    const int32_t* ci = cand_i + (size_t)bg * cstride;
    if (n <= 512) {
      // one wave of ballots (the other three waves have nothing to do here);
      // longer lists are faster through the radix select below
      __shared__ __align__(16) int32_t s_sel[64];
      if (threadIdx.x < 64) {
        wave_topk(cs, ci, 0, n, a.K, nullptr, s_sel);
        wave_lds_sync();
        for (int x = threadIdx.x; x < a.K; x += 64) {
          sl[x] = s_sel[x];
          if (to != nullptr) to[x] = s_sel[x];
        }
      }
    } else if (n <= 256 * PER) {
      select_block<PER>(cs, ci, n, a.K, sl, to);
    } else {
      select_block_big(cs, ci, n, a.K, sl, to);
    }
    return;
  }
  const int x = blk - nbg;
  const int bg = x / wpb;
  const int u = a.K + 4 * (x - bg * wpb) + (threadIdx.x >> 6);
  if (u < a.units) dec_units<T, QT, G, DH, 1, PG>(q, qs, k, v, kL, e, a, bg, u, 1);
}

// the selected-chunk units: wave x of a (sequence, KV head) takes unit x
// (one per wave: at <= 128 VGPRs four waves per SIMD stay resident, which
// measured faster than two units per wave at two waves per SIMD)
template <typename T, typename QT, int G, int DH, bool PG, int NUW>
__global__ __launch_bounds__(256, sizeof(T) == 2 ? (NUW == 1 ? 4 : 2) : 1) void k_dec_chunks(const T* __restrict__ q, const QT* __restrict__ qs,
                                                    const T* __restrict__ k, const T* __restrict__ v,
                                                    const T* __restrict__ kL, const T* __restrict__ e,
                                                    DecArgs a, int wpg) {
  const int x = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (x < wpg) dec_units<T, QT, G, DH, NUW, PG>(q, qs, k, v, kL, e, a, blockIdx.y, x, wpg);
}

// ---------------------------------------------------------------- combine
// one workgroup per (sequence, query head): wave 0 takes the units' maxima
// and weights, then the four waves each sum a quarter of the units' outputs
// (eight units' loads in flight per wave) and wave 0 adds the four parts
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_dec_combine(const float* __restrict__ pml,
                                                     const float* __restrict__ po, T* __restrict__ o,
                                                     float* __restrict__ lse, int Hkv, int G,
                                                     int units) {
  __shared__ float wgt[256];
  __shared__ float part[4][DH];
  __shared__ float stat[2];
  const int bh = blockIdx.x;  // b * Hq + h
  const int Hq = Hkv * G;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / G, hh = h - g * G;
  const int bg = b * Hkv + g;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w == 0) {
    float M = NEG_INF;
    for (int u = lane; u < units; u += 64) M = fmaxf(M, pml[(((size_t)bg * units + u) * G + hh) * 2]);
#pragma unroll
    for (int m2 = 32; m2 >= 1; m2 >>= 1) M = fmaxf(M, __shfl_xor(M, m2, 64));
    float Z = 0.f;
    for (int u = lane; u < units; u += 64) {
      const float* p = pml + (((size_t)bg * units + u) * G + hh) * 2;
      const float m = p[0];
      const float wu = m == NEG_INF ? 0.f : __expf(m - M);
      wgt[u] = wu;
      Z += wu * p[1];
    }
#pragma unroll
    for (int m2 = 32; m2 >= 1; m2 >>= 1) Z += __shfl_xor(Z, m2, 64);
    if (lane == 0) {
      stat[0] = M;
      stat[1] = Z;
    }
  }
  __syncthreads();
  // wave w sums the batches of eight consecutive units starting at 8 w, 8 w + 32, ...
  float acc[DH / 64];
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) acc[j] = 0.f;
  const float* base = po + ((size_t)bg * units * G + hh) * DH;
  for (int u = 8 * w; u < units; u += 32) {
    float x[8][DH / 64];
    // units past the last re-read the last one (in bounds) with weight 0
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int uc = min(u + t, units - 1);
#pragma unroll
      for (int j = 0; j < DH / 64; ++j) x[t][j] = base[(size_t)uc * G * DH + lane + 64 * j];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float wt = u + t < units ? wgt[min(u + t, units - 1)] : 0.f;
#pragma unroll
      for (int j = 0; j < DH / 64; ++j) acc[j] = fmaf(wt, x[t][j], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) part[w][lane + 64 * j] = acc[j];
  __syncthreads();
  if (w == 0) {
    const float Z = stat[1];
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) {
      const int x = lane + 64 * j;
      o[(size_t)bh * DH + x] = from_f<T>((part[0][x] + part[1][x] + part[2][x] + part[3][x]) / Z);
    }
    if (lane == 0) lse[bh] = stat[0] + __logf(Z);
  }
}

// ---------------------------------------------------------------- host side
namespace {
struct DecWs {
  float* qhat;
  float* cand_s;
  int32_t* cand_i;
  int32_t* sel;
  float *pml, *po;
  int nsplit, units, Kc, cstride;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t carve(const Dims& p, void* base, DecWs* w) {
  char* c = static_cast<char*>(base);
  size_t off = 0;
  w->nsplit = std::max(1, (p.C + CPW - 1) / CPW);
  // candidate lists: the top min(K, 512) of every 512 scanned chunks, padded
  // for the selection's vector loads (a multiple of 8, at least 256 * 8)
  w->Kc = std::min(p.K, 512);
  w->cstride = std::max((w->nsplit * 4 * w->Kc + 7) / 8 * 8, 2048);
  w->units = p.K + (p.W + p.S - 1 + 63) / 64 + 1;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + off : nullptr;
    off += up256(bytes);
    return ptr;
  };
  const size_t bg = (size_t)p.B * p.Hkv;
  w->qhat = (float*)take(p.r > 0 ? (size_t)p.B * p.Hq * p.d * sizeof(float) : 0);
  w->cand_s = (float*)take(bg * w->cstride * sizeof(float));
  w->cand_i = (int32_t*)take(bg * w->cstride * sizeof(int32_t));
  w->sel = (int32_t*)take(bg * p.K * sizeof(int32_t));
  w->pml = (float*)take(bg * w->units * p.G * 2 * sizeof(float));
  w->po = (float*)take(bg * w->units * p.G * p.d * sizeof(float));
  return off;
}
}  // namespace

size_t decode_workspace(const Dims& p) {
  DecWs w;
  const size_t s = carve(p, nullptr, &w);
  if (w.units > 256) return (size_t)-1;  // combine weight buffer
  return s;
}

template <typename T, typename QT, int G, int DH, bool PG>
static hipError_t dec_go(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                         const int32_t* seq_len, const int32_t* ptab, int maxp, const void* kL,
                         const void* e, void* o, float* lse, int32_t* topk_idx, const DecWs& w,
                         hipStream_t st) {
  hipLaunchKernelGGL((k_dec_scan<T, QT, G, DH, PG>), dim3(w.nsplit, p.B * p.Hkv), dim3(256), 0, st,
                     (const QT*)qs, (const T*)kL, (const T*)e, seq_len, ptab, maxp, w.cand_s, w.cand_i,
                     w.cstride, w.Kc, p.N, p.C, p.Hkv, p.W, p.S, p.scale);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  DecArgs a;
  a.seq_len = seq_len;
  a.ptab = ptab;
  a.maxp = maxp;
  a.sel = w.sel;
  a.pml = w.pml;
  a.po = w.po;
  a.N = p.N; a.C = p.C; a.Hkv = p.Hkv; a.K = p.K; a.W = p.W; a.S = p.S; a.units = w.units;
  a.scale = p.scale;
  const int nbg = p.B * p.Hkv;
  const int wpb = (w.units - p.K + 3) / 4;  // window units: four per block
  hipLaunchKernelGGL((k_dec_select_window<T, QT, G, DH, 8, PG>), dim3(nbg * (1 + wpb)), dim3(256), 0, st,
                     (const float*)w.cand_s, (const int32_t*)w.cand_i, topk_idx, w.cstride, w.Kc, nbg,
                     wpb, (const T*)q, (const QT*)qs, (const T*)k, (const T*)v, (const T*)kL,
                     (const T*)e, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_chunks<T, QT, G, DH, PG, 1>), dim3((p.K + 3) / 4, nbg), dim3(256), 0, st,
                     (const T*)q, (const QT*)qs, (const T*)k, (const T*)v, (const T*)kL, (const T*)e, a,
                     p.K);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_combine<T, DH>), dim3(p.B * p.Hq), dim3(256), 0, st, (const float*)w.pml,
                     (const float*)w.po, (T*)o, lse, p.Hkv, G, w.units);
  return hipGetLastError();
}

template <typename T, typename QT, int G>
static hipError_t dec_d(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const int32_t* pt, int mp, const void* kL, const void* e,
                        void* o, float* lse, int32_t* idx, const DecWs& w, hipStream_t st) {
  if (pt != nullptr) {
    if (p.d == 64) return dec_go<T, QT, G, 64, true>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
    return dec_go<T, QT, G, 128, true>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
  }
  if (p.d == 64) return dec_go<T, QT, G, 64, false>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
  return dec_go<T, QT, G, 128, false>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
}

template <typename T, typename QT>
static hipError_t dec_g(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const int32_t* pt, int mp, const void* kL, const void* e,
                        void* o, float* lse, int32_t* idx, const DecWs& w, hipStream_t st) {
  switch (p.G) {
    case 1: return dec_d<T, QT, 1>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
    case 2: return dec_d<T, QT, 2>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
    case 4: return dec_d<T, QT, 4>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
    case 8: return dec_d<T, QT, 8>(p, qs, q, k, v, sl, pt, mp, kL, e, o, lse, idx, w, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Dims& p, const void* qs, bool q_is_f32, const void* q, const void* k,
                         const void* v, const int32_t* seq_len, const int32_t* page_table,
                         int max_pages, const void* kL, const void* e, void* o, float* lse,
                         int32_t* topk_idx, void* ws, hipStream_t st) {
  DecWs w;
  carve(p, ws, &w);
  const int32_t* pt = page_table;
  const int mp = max_pages;
  if (p.dtype == 1) {
    if (q_is_f32) return dec_g<uint16_t, float>(p, qs, q, k, v, seq_len, pt, mp, kL, e, o, lse, topk_idx, w, st);
    return dec_g<uint16_t, uint16_t>(p, qs, q, k, v, seq_len, pt, mp, kL, e, o, lse, topk_idx, w, st);
  }
  return dec_g<float, float>(p, qs, q, k, v, seq_len, pt, mp, kL, e, o, lse, topk_idx, w, st);
}

}  // namespace hils
