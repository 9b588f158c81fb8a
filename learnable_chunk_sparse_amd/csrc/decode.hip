// HiLS decode step: one new query per sequence (paper Fig. 6 decode latency;
// nestfrontier "The routing problem": score the chunk summaries, keep the top
// K distant chunks, attend inside them and in the local window).
//
// The step is bound by HBM bandwidth: every distant landmark key is read once
// (the O(L/S) per-token retrieval term), then only the K selected chunks and
// the window. Four launches:
//   k_dec_scan    streaming landmark scan: each workgroup scores CPW chunks of
//                 one (sequence, KV head) with 16x16x32 MFMAs (rows = chunks,
//                 columns = the group's heads, hi and lo halves of the fp32
//                 query), takes the max over heads and stores the score.
//   k_dec_select  per (sequence, KV head): the K-th largest score by a 4-pass
//                 8-bit radix select over order-preserving integer keys, ties
//                 resolved by lower chunk index, and the chosen ids written in
//                 ascending order by a prefix sum (no sort).
//   k_dec_attn    one wave per 64-token unit (a selected chunk or a window
//                 block) for all G heads: S^T = K Q^T on MFMA, softmax, O^T =
//                 V^T P^T; the V^T operands come from the row-major V
//                 fragments by a product with the identity (exact), so nothing
//                 is staged in LDS. A chunk unit leaves (log-weight s_c,
//                 weight 1, O_c); a window block leaves its (max, sum,
//                 unnormalised output).
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
// exclusive prefix sum of v over the 1024 threads of the block; total as well
__device__ __forceinline__ int block_scan1024(int v, int* wsum, int& total) {
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
  for (int j = 0; j < 16; ++j) {
    const int s2 = wsum[j];
    base += j < w ? s2 : 0;
    tot += s2;
  }
  __syncthreads();
  total = tot;
  return base + x - v;
}

// The K largest scores of one (sequence, KV head) by (score desc, index asc),
// written as ascending chunk ids, -1 padded.
__global__ __launch_bounds__(1024) void k_dec_select(const float* __restrict__ scores,
                                                     const int32_t* __restrict__ seq_len,
                                                     int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ topk_out, int N, int Cp,
                                                     int Hkv, int K, int W, int S) {
  __shared__ int hist[256];
  __shared__ int wsum[16];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_krem;
  const int t = threadIdx.x;
  const int bg = blockIdx.x, b = bg / Hkv;
  const int nd = n_distant(seq_n(seq_len, b, N) - 1, W, S);
  const float* src = scores + (size_t)bg * Cp;
  const bool take_all = nd <= K;
  if (t == 0) {
    s_prefix = 0u;
    s_mask = 0u;
    s_krem = K;
  }
  __syncthreads();
  // radix select: the exact key T of the K-th largest score, and how many of
  // the keys equal to T are taken (krem)
  if (!take_all) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (t < 256) hist[t] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int c = t; c < nd; c += 1024) {
        const uint32_t key = ord_f(src[c]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
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
  }
  const uint32_t T = s_prefix;
  const int krem = s_krem;
  // contiguous index ranges per thread, so that prefix sums follow index order
  const int per = (nd + 1023) / 1024;
  const int lo = min(nd, t * per), hi = min(nd, lo + per);
  int ties = 0;
  if (!take_all)
    for (int c = lo; c < hi; ++c) ties += ord_f(src[c]) == T;
  int tot;
  const int tie0 = block_scan1024(ties, wsum, tot);
  auto taken = [&](int c, int& tr) {
    if (take_all) return true;
    const uint32_t key = ord_f(src[c]);
    const bool tk = key > T || (key == T && tr < krem);
    tr += key == T;
    return tk;
  };
  int cnt = 0;
  {
    int tr = tie0;
    for (int c = lo; c < hi; ++c) cnt += taken(c, tr) ? 1 : 0;
  }
  const int out0 = block_scan1024(cnt, wsum, tot);
  {
    int tr = tie0, o = out0;
    for (int c = lo; c < hi; ++c) {
      if (taken(c, tr)) {
        sel[(size_t)bg * K + o] = c;
        if (topk_out != nullptr) topk_out[(size_t)bg * K + o] = c;
        ++o;
      }
    }
  }
  for (int k2 = tot + t; k2 < K; k2 += 1024) {
    sel[(size_t)bg * K + k2] = -1;
    if (topk_out != nullptr) topk_out[(size_t)bg * K + k2] = -1;
  }
}

// ---------------------------------------------------------------- attention units
// partials per (bg, unit, head): pml = [m, l], po = U[0..DH)
template <typename T, typename QT, int G, int DH>
__global__ __launch_bounds__(256) void k_dec_attn(const T* __restrict__ q, const QT* __restrict__ qs,
                                                  const T* __restrict__ k, const T* __restrict__ v,
                                                  const T* __restrict__ kL, const T* __restrict__ e,
                                                  const int32_t* __restrict__ seq_len,
                                                  const int32_t* __restrict__ sel,
                                                  float* __restrict__ pml, float* __restrict__ po,
                                                  int N, int C, int Hkv, int K, int W, int S,
                                                  float scale, int units) {
  typedef typename Frag<T>::type FT;
  constexpr int KS = DH / 32, MB = DH / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int gl = lane >> 4, col = lane & 15;
  const int u = blockIdx.x * 4 + w;
  const int bg = blockIdx.y;
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
  w->Cp = w->nsplit * CPW;
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
  hipLaunchKernelGGL(k_dec_select, dim3(p.B * p.Hkv), dim3(1024), 0, st, (const float*)w.scores,
                     seq_len, w.sel, topk_idx, p.N, w.Cp, p.Hkv, p.K, p.W, p.S);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((k_dec_attn<T, QT, G, DH>), dim3((w.units + 3) / 4, p.B * p.Hkv), dim3(256), 0,
                     st, (const T*)q, (const QT*)qs, (const T*)k, (const T*)v, (const T*)kL,
                     (const T*)e, seq_len, w.sel, w.pml, w.po, p.N, p.C, p.Hkv, p.K, p.W, p.S,
                     p.scale, w.units);
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
