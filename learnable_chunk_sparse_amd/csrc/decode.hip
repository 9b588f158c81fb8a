// HiLS decode step: one new query per sequence (paper Fig. 6 decode latency;
// nestfrontier "The routing problem": score the chunk summaries, keep the top
// K distant chunks, attend inside them and in the local window).
//
// The step is bound by HBM bandwidth: every distant landmark key is read once
// (the O(L/S) per-token retrieval term), then only the K selected chunks and
// the window. Four launches:
//   k_dec_scan    streaming landmark scan: each wave scores CPW/4 chunks of
//                 one (sequence, KV head) with 16x16x32 MFMAs (rows = the
//                 group's query heads, hi and lo halves of an fp32 query;
//                 columns = chunks), a ring of four 16-chunk steps in flight;
//                 the max over heads is in-lane; scores go out through LDS.
//   k_dec_select_window
//                 blocks 0 .. B Hkv - 1: the top-K of one (sequence, KV head)
//                 by a 4-pass 8-bit radix select over order-preserving integer
//                 keys held in registers, ties resolved by lower chunk index,
//                 the chosen ids written in ascending order by a prefix sum (no
//                 sort). The other blocks run the window units, which do not
//                 depend on the selection and keep HBM busy meanwhile.
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

// ---------------------------------------------------------------- scan
// D[head][chunk] = q_h . kL_c: the query heads are the A operand (rows; hi
// and lo bf16 halves of an fp32 query accumulate into the same product), the
// landmark rows the B operand (columns), so lane (g, c) ends with the scores
// of chunk c for heads 4 g .. 4 g + 3 and the max over heads is in-lane.
template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_dec_scan(const QT* __restrict__ qs, const T* __restrict__ kL,
                                                  const T* __restrict__ e,
                                                  const int32_t* __restrict__ seq_len,
                                                  float* __restrict__ scores, int N, int C, int Cp,
                                                  int Hkv, int W, int S, float scale) {
  typedef typename Frag<T>::type FT;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  constexpr int KS = DH / 32;
  constexpr int NST = CPW / 64;  // 16-chunk steps per wave
  constexpr int PD = 4;          // steps in flight per wave
  static_assert(G <= 8 && NST % PD == 0, "scan shape");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int gl = lane >> 4, col = lane & 15;
  const int split = blockIdx.x, bg = blockIdx.y;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int n = seq_n(seq_len, b, N);
  const int nd = n_distant(n - 1, W, S);
  const int c_w = split * CPW + (CPW / 4) * w;  // this wave's first chunk
  if (c_w >= nd) return;
  const T* kLg = kL + (size_t)bg * C * DH;
  const T* eg = e + (size_t)bg * C;
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
    const int c = min(cstep(st) + col, nd - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kd[ks] = ld8<T>(kLg + (size_t)c * DH + 8 * gl + 32 * ks);
    ed = to_f<T>(eg[c]);
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
  // scores are collected in LDS and written once per wave as whole lines
  // (scattered 64-byte stores between the reads cost ~10% of the scan)
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
  float* dst = scores + (size_t)bg * Cp + c_w;
#pragma unroll
  for (int x = 0; x < CPW / 4 / 256; ++x) {
    const int o = 4 * (lane + 64 * x);
    *reinterpret_cast<f32x4*>(dst + o) = *reinterpret_cast<const f32x4*>(sw + o);
  }
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

// The K largest scores of one (sequence, KV head) by (score desc, index asc),
// written as ascending chunk ids, -1 padded; one 256-thread block. Thread t
// holds the order-preserving integer keys of chunks [t PER, t PER + PER) in
// registers (contiguous ranges, so prefix sums follow index order); the exact
// key T of the K-th largest score comes from a 4-pass 8-bit radix select,
// and krem of the keys equal to T (the lowest indices) are taken.
template <int PER>
__device__ __forceinline__ void select_block(const float* __restrict__ src, int nd, int K,
                                             int32_t* __restrict__ sel, int32_t* __restrict__ topk_out) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem;
  const int t = threadIdx.x;
  const int lo = t * PER;
  // vector loads (the score buffer is padded to at least 256 PER entries);
  // key 0 marks a slot past the last distant chunk (no finite score maps to 0)
  uint32_t key[PER];
#pragma unroll
  for (int j4 = 0; j4 < PER / 4; ++j4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + lo + 4 * j4);
#pragma unroll
    for (int i = 0; i < 4; ++i) key[4 * j4 + i] = lo + 4 * j4 + i < nd ? ord_f(x[i]) : 0u;
  }
  const bool take_all = nd <= K;
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
      // neighbouring chunks mostly share the high digits: runs of one bin are
      // added at once (far fewer lanes hit one LDS address per instruction)
      int pb = -1, pc = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        if (key[j] != 0u && (key[j] & mask) == prefix) {
          const int bin = (key[j] >> shift) & 255;
          if (bin != pb) {
            if (pc > 0) atomicAdd(&hist[pb], pc);
            pb = bin;
            pc = 0;
          }
          ++pc;
        }
      }
      if (pc > 0) atomicAdd(&hist[pb], pc);
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
  int tot;
  const int tie0 = block_scan256(ties, wsum, tot);
  // chunk lo + j is taken: above T, or equal to T among the first krem ties
  // (tr counts the ties before it)
  auto taken = [&](int j, int& tr) __attribute__((always_inline)) {
    const bool valid = key[j] != 0u;
    const bool eq = !take_all && key[j] == T;
    const bool tk = valid && (take_all || key[j] > T || (eq && tr < krem));
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
        sel[o] = lo + j;
        if (topk_out != nullptr) topk_out[o] = lo + j;
        ++o;
      }
    }
  }
  for (int k2 = tot + t; k2 < K; k2 += 256) {
    sel[k2] = -1;
    if (topk_out != nullptr) topk_out[k2] = -1;
  }
}

// larger chunk counts: keys re-read from the score buffer on every pass,
// eight per thread and iteration (the buffer is padded to a multiple of 2048)
__device__ __forceinline__ void select_block_big(const float* __restrict__ src, int nd, int K,
                                                 int32_t* __restrict__ sel, int32_t* __restrict__ topk_out) {
  __shared__ int hist[256];
  __shared__ int wsum[4];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem;
  const int t = threadIdx.x;
  const bool take_all = nd <= K;
  if (t == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_krem = K;
  }
  __syncthreads();
  auto keys8 = [&](int c0, uint32_t (&kk)[8]) __attribute__((always_inline)) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(src + c0);
    const f32x4 b2 = *reinterpret_cast<const f32x4*>(src + c0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kk[i] = c0 + i < nd ? ord_f(a[i]) : 0u;
      kk[4 + i] = c0 + 4 + i < nd ? ord_f(b2[i]) : 0u;
    }
  };
  if (!take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[t] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int c0 = 8 * t; c0 < nd; c0 += 2048) {
        uint32_t kk[8];
        keys8(c0, kk);
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
  // contiguous ranges of a multiple of 8 chunks per thread (prefix sums follow
  // index order)
  const int per = ((nd + 255) / 256 + 7) / 8 * 8;
  const int lo = min(nd, t * per), hi = min(nd, lo + per);
  int ties = 0;
  if (!take_all)
    for (int c0 = lo; c0 < hi; c0 += 8) {
      uint32_t kk[8];
      keys8(c0, kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) ties += kk[i] == T ? 1 : 0;
    }
  int tot;
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
      keys8(c0, kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) cnt += taken(kk[i], tr) ? 1 : 0;
    }
  }
  const int out0 = block_scan256(cnt, wsum, tot);
  {
    int tr = tie0, o = out0;
    for (int c0 = lo; c0 < hi; c0 += 8) {
      uint32_t kk[8];
      keys8(c0, kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (taken(kk[i], tr)) {
          sel[o] = c0 + i;
          if (topk_out != nullptr) topk_out[o] = c0 + i;
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
  const int32_t* sel;
  float *pml, *po;
  int N, C, Hkv, K, W, S, units;
  float scale;
};

// one wave: unit u of (sequence, KV head) bg
template <typename T, typename QT, int G, int DH>
__device__ __forceinline__ void dec_unit(const T* __restrict__ q, const QT* __restrict__ qs,
                                         const T* __restrict__ k, const T* __restrict__ v,
                                         const T* __restrict__ kL, const T* __restrict__ e,
                                         const DecArgs& a, int bg, int u) {
  typedef typename Frag<T>::type FT;
  constexpr int KS = DH / 32, MB = DH / 16;
  const int lane = threadIdx.x & 63;
  const int gl = lane >> 4, col = lane & 15;
  const int32_t* seq_len = a.seq_len;
  const int32_t* sel = a.sel;
  float* pml = a.pml;
  float* po = a.po;
  const int N = a.N, C = a.C, Hkv = a.Hkv, K = a.K, W = a.W, S = a.S, units = a.units;
  const float scale = a.scale;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  if (u >= units) return;
  const int n = seq_n(seq_len, b, N);
  const int i = n - 1;
  const int nd = n_distant(i, W, S);
  const int ws = nd * S;
  float* pm = pml + ((size_t)bg * units + u) * G * 2;
  float* pv = po + ((size_t)bg * units + u) * G * DH;
  // what this unit covers
  int t0, cnt, chunk = -1;
  if (u < K) {
    chunk = sel[(size_t)bg * K + u];
    t0 = chunk * S;
    cnt = chunk >= 0 ? S : 0;
  } else {
    t0 = ws + 64 * (u - K);
    cnt = min(64, n - t0);
  }
  if (cnt <= 0) {
    // an empty unit: weight 0 and a zero vector (the combine multiplies
    // every unit's vector by its weight without branching)
    if (lane < G) {
      pm[2 * lane] = NEG_INF;
      pm[2 * lane + 1] = 0.f;
    }
    for (int x = lane; x < G * DH / 4; x += 64) reinterpret_cast<f32x4*>(pv)[x] = zero4();
    return;
  }
  // K and V rows as row-major fragments: token 16 tb + col, dims 8 gl + 32 ks
  const T* kb = k + ((size_t)bg * N + t0) * DH;
  const T* vb = v + ((size_t)bg * N + t0) * DH;
  FT kf[4][KS], vf[4][KS];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    int tok = 16 * tb + col;
    tok = tok < cnt ? tok : 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[tb][ks] = ld8<T>(kb + (size_t)tok * DH + 8 * gl + 32 * ks);
      vf[tb][ks] = ld8<T>(vb + (size_t)tok * DH + 8 * gl + 32 * ks);
    }
  }
  // Q^T operand: column col = head col (raw query), zero beyond G
  FT qf[KS];
  {
    const int h = col < G ? col : 0;
    const T* src = q + ((size_t)b * Hq + g * G + h) * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const FT raw = ld8<T>(src + 32 * ks);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = col < G ? (float)raw[j] : 0.f;
      qf[ks] = pack8<T>(x);
    }
  }
  // per-head fusion score of a selected chunk: s_h = scale q_hat_h . kL_c + e_c
  float s_head[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s_head[h] = 0.f;
  if (chunk >= 0) {
    const T* kr = kL + ((size_t)bg * C + chunk) * DH;
    const float eb = to_f<T>(e[(size_t)bg * C + chunk]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const QT* qh = qs + ((size_t)b * Hq + g * G + h) * DH;
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < DH / 64; ++j) a = fmaf(to_f<QT>(qh[lane + 64 * j]), to_f<T>(kr[lane + 64 * j]), a);
#pragma unroll
      for (int m2 = 32; m2 >= 1; m2 >>= 1) a += __shfl_xor(a, m2, 64);
      s_head[h] = fmaf(a, scale, eb);
    }
  }
  f32x4 sacc[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    sacc[tb] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc[tb] = mma16(kf[tb][ks], qf[ks], sacc[tb]);
  }
  float mx = NEG_INF;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int tok = 16 * tb + 4 * gl + ii;
      const float x = tok < cnt ? sacc[tb][ii] * scale : NEG_INF;
      sacc[tb][ii] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
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
  ls += shfl_xor(ls, 16);
  ls += shfl_xor(ls, 32);
  // identity fragments: I_h[k][c] = (k == 16 h + c)
  FT idf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (8 * gl + j == 16 * h + col) ? 1.f : 0.f;
    idf[h] = pack8<T>(x);
  }
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
  if (col < G) {
    float mval = mx, lval = ls, coef = 1.f;
    if (chunk >= 0) {
      // a selected chunk enters the fusion as one term: log-weight s_c,
      // weight 1, vector O_c
      float sh = s_head[0];
#pragma unroll
      for (int h = 1; h < G; ++h) sh = col == h ? s_head[h] : sh;
      mval = sh;
      lval = 1.f;
      coef = 1.f / ls;
    }
    if (gl == 0) {
      pm[2 * col] = mval;
      pm[2 * col + 1] = lval;
    }
    float* ph = pv + (size_t)col * DH + 4 * gl;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *reinterpret_cast<f32x4*>(ph + 16 * mb) = oacc[mb] * coef;
  }
}

// selections (one block per (sequence, KV head)) and, alongside in the same
// launch, the window units, which do not depend on them
template <typename T, typename QT, int G, int DH, int PER>
__global__ __launch_bounds__(256) void k_dec_select_window(const float* __restrict__ scores,
                                                           int32_t* __restrict__ topk_out, int Cp,
                                                           int nbg, int wpb, const T* __restrict__ q,
                                                           const QT* __restrict__ qs,
                                                           const T* __restrict__ k,
                                                           const T* __restrict__ v,
                                                           const T* __restrict__ kL,
                                                           const T* __restrict__ e, DecArgs a) {
  const int blk = blockIdx.x;
  if (blk < nbg) {
    const int bg = blk, b = bg / a.Hkv;
    const int nd = n_distant(seq_n(a.seq_len, b, a.N) - 1, a.W, a.S);
    int32_t* sl = const_cast<int32_t*>(a.sel) + (size_t)bg * a.K;
    int32_t* to = topk_out != nullptr ? topk_out + (size_t)bg * a.K : nullptr;
    if (nd <= 256 * PER)
      select_block<PER>(scores + (size_t)bg * Cp, nd, a.K, sl, to);
    else
      select_block_big(scores + (size_t)bg * Cp, nd, a.K, sl, to);
    return;
  }
  const int x = blk - nbg;
  const int bg = x / wpb;
  const int u = a.K + 4 * (x - bg * wpb) + (threadIdx.x >> 6);
  if (u < a.units) dec_unit<T, QT, G, DH>(q, qs, k, v, kL, e, a, bg, u);
}

// the selected-chunk units
template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_dec_chunks(const T* __restrict__ q, const QT* __restrict__ qs,
                                                    const T* __restrict__ k, const T* __restrict__ v,
                                                    const T* __restrict__ kL, const T* __restrict__ e,
                                                    DecArgs a) {
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u < a.K) dec_unit<T, QT, G, DH>(q, qs, k, v, kL, e, a, blockIdx.y, u);
}

// ---------------------------------------------------------------- combine
// one wave per (sequence, query head): lanes first take units (max, weights),
// then dims (the weighted sum, eight units' loads in flight at a time)
template <typename T, int DH>
__global__ __launch_bounds__(64) void k_dec_combine(const float* __restrict__ pml,
                                                    const float* __restrict__ po, T* __restrict__ o,
                                                    float* __restrict__ lse, int Hkv, int G,
                                                    int units) {
  __shared__ float wgt[256];
  const int bh = blockIdx.x;  // b * Hq + h
  const int Hq = Hkv * G;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / G, hh = h - g * G;
  const int bg = b * Hkv + g;
  const int lane = threadIdx.x;
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
  __syncthreads();
  float acc[DH / 64];
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) acc[j] = 0.f;
  const float* base = po + ((size_t)bg * units * G + hh) * DH;
  int u = 0;
  for (; u + 8 <= units; u += 8) {
    float x[8][DH / 64];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < DH / 64; ++j) x[t][j] = base[(size_t)(u + t) * G * DH + lane + 64 * j];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < DH / 64; ++j) acc[j] = fmaf(wgt[u + t], x[t][j], acc[j]);
  }
  for (; u < units; ++u)
#pragma unroll
    for (int j = 0; j < DH / 64; ++j) acc[j] = fmaf(wgt[u], base[(size_t)u * G * DH + lane + 64 * j], acc[j]);
#pragma unroll
  for (int j = 0; j < DH / 64; ++j) o[(size_t)bh * DH + lane + 64 * j] = from_f<T>(acc[j] / Z);
  if (lane == 0) lse[bh] = M + __logf(Z);
}

// ---------------------------------------------------------------- host side
namespace {
struct DecWs {
  float* qhat;
  float* scores;
  int32_t* sel;
  float *pml, *po;
  int nsplit, units, Cp;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t carve(const Dims& p, void* base, DecWs* w) {
  char* c = static_cast<char*>(base);
  size_t off = 0;
  w->nsplit = std::max(1, (p.C + CPW - 1) / CPW);
  // scores padded for the selection's vector loads: a multiple of 2048 and
  // at least 256 * 32 (one register set of keys per thread)
  w->Cp = std::max(w->nsplit * CPW, 8192);
  w->units = p.K + (p.W + p.S - 1 + 63) / 64 + 1;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + off : nullptr;
    off += up256(bytes);
    return ptr;
  };
  const size_t bg = (size_t)p.B * p.Hkv;
  w->qhat = (float*)take(p.r > 0 ? (size_t)p.B * p.Hq * p.d * sizeof(float) : 0);
  w->scores = (float*)take(bg * w->Cp * sizeof(float));
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

template <typename T, typename QT, int G, int DH>
static hipError_t dec_go(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                         const int32_t* seq_len, const void* kL, const void* e, void* o, float* lse,
                         int32_t* topk_idx, const DecWs& w, hipStream_t st) {
  hipLaunchKernelGGL((k_dec_scan<T, QT, G, DH>), dim3(w.nsplit, p.B * p.Hkv), dim3(256), 0, st,
                     (const QT*)qs, (const T*)kL, (const T*)e, seq_len, w.scores, p.N, p.C, w.Cp,
                     p.Hkv, p.W, p.S, p.scale);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  DecArgs a;
  a.seq_len = seq_len;
  a.sel = w.sel;
  a.pml = w.pml;
  a.po = w.po;
  a.N = p.N; a.C = p.C; a.Hkv = p.Hkv; a.K = p.K; a.W = p.W; a.S = p.S; a.units = w.units;
  a.scale = p.scale;
  const int nbg = p.B * p.Hkv;
  const int wpb = (w.units - p.K + 3) / 4;  // window units: four per block
  hipLaunchKernelGGL((k_dec_select_window<T, QT, G, DH, 32>), dim3(nbg * (1 + wpb)), dim3(256), 0, st,
                     (const float*)w.scores, topk_idx, w.Cp, nbg, wpb, (const T*)q, (const QT*)qs,
                     (const T*)k, (const T*)v, (const T*)kL, (const T*)e, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_chunks<T, QT, G, DH>), dim3((p.K + 3) / 4, nbg), dim3(256), 0, st,
                     (const T*)q, (const QT*)qs, (const T*)k, (const T*)v, (const T*)kL, (const T*)e, a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_combine<T, DH>), dim3(p.B * p.Hq), dim3(64), 0, st, (const float*)w.pml,
                     (const float*)w.po, (T*)o, lse, p.Hkv, G, w.units);
  return hipGetLastError();
}

template <typename T, typename QT, int G>
static hipError_t dec_d(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const void* kL, const void* e, void* o, float* lse,
                        int32_t* idx, const DecWs& w, hipStream_t st) {
  if (p.d == 64) return dec_go<T, QT, G, 64>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
  return dec_go<T, QT, G, 128>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
}

template <typename T, typename QT>
static hipError_t dec_g(const Dims& p, const void* qs, const void* q, const void* k, const void* v,
                        const int32_t* sl, const void* kL, const void* e, void* o, float* lse,
                        int32_t* idx, const DecWs& w, hipStream_t st) {
  switch (p.G) {
    case 1: return dec_d<T, QT, 1>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 2: return dec_d<T, QT, 2>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 4: return dec_d<T, QT, 4>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    case 8: return dec_d<T, QT, 8>(p, qs, q, k, v, sl, kL, e, o, lse, idx, w, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const Dims& p, const void* qs, bool q_is_f32, const void* q, const void* k,
                         const void* v, const int32_t* seq_len, const void* kL, const void* e,
                         void* o, float* lse, int32_t* topk_idx, void* ws, hipStream_t st) {
  DecWs w;
  carve(p, ws, &w);
  if (p.dtype == 1) {
    if (q_is_f32) return dec_g<uint16_t, float>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
    return dec_g<uint16_t, uint16_t>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
  }
  return dec_g<float, float>(p, qs, q, k, v, seq_len, kL, e, o, lse, topk_idx, w, st);
}

}  // namespace hils
