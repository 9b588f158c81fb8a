// Routing: surrogate chunk scores, GQA max over the group's heads and a
// running top-K, fused so that the O(N^2 / S) score matrix never leaves the
// chip (paper: surrogate-score step of "The HiLS-Attention Mechanism", the
// GQA max paragraph, top-K selection; nestfrontier "The routing problem" for
// the O(N^2/S) routing term).
//
//   s_{h,c}(i) = scale * q_hat_h(i) . kL_c + e_c  for c < n_dist(i)
//   sel_c(i)   = max_{h in group} s_{h,c}(i)
//   T(i)       = the K best c by (sel desc, c asc)
//
// Workgroup = 4 waves of 16 * RB consecutive positions of one (batch, KV head)
// (RB = 4 / G row groups, so that a wave's MFMA rows are 64 (position, head)
// pairs for G <= 4). Landmark keys stream
// through LDS in tiles of 64 chunks shared by the four waves (the next tile
// is prefetched into registers while the current one is scored). Scores come
// from 16x16x32 bf16 MFMAs: the fp32 q_hat is split into hi + lo bf16 parts
// (two products with fp32 accumulation; landmark keys are exact bf16), which
// keeps each score within ~1e-6 of its fp64 value.
// Selection: the max-over-heads score tile of each 16-chunk step is turned
// around through LDS so that one lane holds one position's 16 candidates, and
// each lane keeps its own running top-K in registers (see TopK below).
#include "hils_common.h"
#include "hils_internal.h"

namespace hils {

namespace {
constexpr int RT_TC = 64;   // chunks per LDS tile
constexpr int RT_PAD = 8;   // kL tile row padding (elements)

}  // namespace

// One lane per position keeps that position's running top-KC (KC >= K) in
// registers as keys, sorted descending: the order-preserving bits of the
// score above the complement of the chunk id, so that one comparison orders
// by (score desc, chunk asc) and 0 lies below every real candidate. A
// candidate that does not beat the running K-th key can never enter the final
// top-K, so each step only appends the candidates that do to a per-lane buffer
// in LDS (one compare and one LDS write per candidate); once the K-th key has
// settled few candidates pass. When a buffer could overflow, every lane's
// buffer is sorted 16 at a time by a bitonic network and merged into its list
// in one pass (a half-cleaner against the current list, then a bitonic merge),
// and the K-th key is refreshed.
// The key is that integer held exactly in a double: the order-preserving 32
// bits of the score times 2^20 plus (2^20 - 1 - chunk), below 2^52 for the
// at most 2^20 chunks a call may have, so that a compare-exchange is one fp64
// max and one fp64 min (a 64-bit integer one took a compare, four selects and
// two hazard waits).
typedef double Key;
constexpr double KEY_CH = 1048576.0;  // 2^20: chunk ids below it
constexpr int SELBUF = 32;            // buffered candidates per position (a multiple of 16)
__device__ __forceinline__ Key sel_key(float sc, int c) {
  const uint32_t u = __float_as_uint(sc);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return fma((double)o, KEY_CH, (double)(1048575 - c));
}
__device__ __forceinline__ float key_score(Key k) {
  const uint32_t o = (uint32_t)((uint64_t)k >> 20);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int key_chunk(Key k) { return 1048575 - (int)((uint64_t)k & 0xFFFFFu); }

// a keeps the larger key when desc, the smaller otherwise
__device__ __forceinline__ void cex(Key& a, Key& b, bool desc) {
  const Key hi = fmax(a, b), lo = fmin(a, b);
  a = desc ? hi : lo;
  b = desc ? lo : hi;
}

template <int NS>
__device__ __forceinline__ void bitonic_sort_desc(Key (&a)[NS]) {
#pragma unroll
  for (int k = 2; k <= NS; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int l = i ^ j;
        if (l > i) cex(a[i], a[l], (i & k) == 0);
      }
}

// t (KC keys, descending) := the KC largest of t and n (16 keys, descending)
template <int KC>
__device__ __forceinline__ void merge_top(Key (&t)[KC], const Key (&n)[16]) {
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int m = KC - 1 - i;
    if (m < 16) t[i] = fmax(n[m], t[i]);
  }
#pragma unroll
  for (int j = KC >> 1; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int l = i ^ j;
      if (l > i) cex(t[i], t[l], true);
    }
}

// UR > 0 (bf16, one head per KV head, Q-Cal rank r = 32 UR): the calibrated
// query is never formed. Since q_hat . kL = q . kL + u . (W_up^T kL), the A
// operand is the raw query (exact bf16) followed by the fp32 u = W_down h
// (hi + lo halves), and the B operand the landmark key followed by the
// precomputed W_up^T kL (hi + lo planes, k_route_klp): three more products
// per k step of r, and no fp32 q_hat written or read.
// Selection mode: SM 0 merges each step's candidates into the lists (one lane
// per position, after the score tile is turned around through LDS), for a
// short scan where most candidates enter the lists anyway; SM 2 (grouped
// heads, or long scans) filters the candidates in the MFMA output layout
// itself, every lane holding 4 RB candidates of a step, against a float
// threshold per position, and appends the few that pass to their position's
// buffer at ranks taken from ballots.
template <typename T, typename QT, int G, int DH, int KC, int UR, bool BUFSEL>
__global__ __launch_bounds__(256, (UR > 0 || (G >= 2 && KC <= 16)) ? 2 : 1) void k_route(const QT* __restrict__ qs, const T* __restrict__ kL,
                                               const T* __restrict__ e, int32_t* __restrict__ topk_idx,
                                               float* __restrict__ topk_score,
                                               float* __restrict__ sel_lse, int N, int C, int Hkv,
                                               int K, int W, int S, float scale, int ntiles,
                                               const float* __restrict__ uq,
                                               const uint16_t* __restrict__ klh,
                                               const uint16_t* __restrict__ kll) {
  static_assert(UR == 0 || (G == 1 && sizeof(T) == 2 && sizeof(QT) == 2), "u path: bf16, G = 1");
  typedef typename Frag<T>::type FT;
  constexpr bool HAS_LO = (sizeof(T) == 2) && (sizeof(QT) == 4);
  constexpr int KS = DH / 32;
  constexpr int KP = DH + RT_PAD;
  constexpr int RB = G >= 4 ? 1 : 4 / G;   // 16-position row groups per wave
  constexpr int PW = 16 * RB;              // positions per wave
  constexpr int PWG = 4 * PW;              // positions per workgroup
  constexpr int TILE_ELEMS = RT_TC * DH;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int NV = TILE_ELEMS / 256 / VEC;
  __shared__ __align__(16) T kl_s[RT_TC * KP];
  __shared__ __align__(16) float e_s[RT_TC];
  constexpr int URN = UR > 0 ? UR : 1, RR = 32 * URN, RP = RR + 8;
  __shared__ __align__(16) uint16_t klh_s[UR ? RT_TC * RP : 8], kll_s[UR ? RT_TC * RP : 8];
  constexpr int SM = G >= 2 ? 2 : (BUFSEL ? 1 : 0);
  static_assert(SM != 1 || PW == 64, "SM 1: one position per lane");
  // per-wave score tile (positions x chunks) for the turnaround (SM 0, SM 1)
  __shared__ __align__(16) float sc_s[SM == 2 ? 1 : 4][SM == 2 ? 1 : PW][16 + 4];
  // per-position buffers of candidates that beat the running K-th key
  // (slot-major: position p's slot j at [j][p]); SM 2 also passes counts and
  // K-th keys between the output layout and the owner lanes. SM 1 flushes as
  // soon as a buffer is full, also inside a step, so 16 slots do.
  constexpr int SB = SM == 1 ? 16 : SELBUF;
  __shared__ float cbs_s[SM ? 4 : 1][SM ? SB : 1][SM ? PW : 1];  // buffered scores
  __shared__ int cbc_s[SM ? 4 : 1][SM ? SB : 1][SM ? PW : 1];    // and their chunks
  __shared__ float thr_s[SM == 2 ? 4 : 1][SM == 2 ? PW : 1];
  __shared__ int cnt_s[SM == 2 ? 4 : 1][SM == 2 ? PW : 1];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int grp = lane >> 4, col = lane & 15;
  const int tile = ntiles - 1 - blockIdx.x;      // heavy (late) tiles first
  const int bg = blockIdx.y;                     // b * Hkv + g
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int pw0 = tile * PWG + w * PW;           // first position of this wave

  // A fragments: row block rb = 16 positions (pw0 + 16 rb + lane%16), per head
  FT ahi[RB][G][KS];
  FT alo[RB][G][HAS_LO ? KS : 1];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int pos = pw0 + 16 * rb + col;
    pos = pos < N ? pos : N - 1;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const QT* src = qs + (((size_t)b * Hq + g * G + hh) * N + pos) * DH + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = to_f<QT>(src[32 * ks + j]);
        ahi[rb][hh][ks] = pack8<T>(x);
        if constexpr (HAS_LO) {
          const u16x8 hb = __builtin_bit_cast(u16x8, ahi[rb][hh][ks]);
          float y[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) y[j] = x[j] - bf2f(hb[j]);
          alo[rb][hh][ks] = pack8<T>(y);
        }
      }
    }
  }
  // u fragments (u path): rows as above, k = the head's r entries of u
  FT uhi[RB][URN], ulo[RB][URN];
  if constexpr (UR > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      int pos = pw0 + 16 * rb + col;
      pos = pos < N ? pos : N - 1;
      const float* src = uq + ((size_t)b * N + pos) * (size_t)Hq * RR + (size_t)g * RR + 8 * grp;
#pragma unroll
      for (int kr = 0; kr < UR; ++kr) {
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(src + 32 * kr);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 32 * kr + 4);
        float x[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        uhi[rb][kr] = pack8<T>(x);
        const u16x8 hb = __builtin_bit_cast(u16x8, uhi[rb][kr]);
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = x[j] - bf2f(hb[j]);
        ulo[rb][kr] = pack8<T>(y);
      }
    }
  }
  // selection state: lane p < PW owns position pw0 + p
  const int mypos = pw0 + lane;
  const int mynd = (lane < PW && mypos < N) ? n_distant(mypos, W, S) : 0;
  Key tk[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) tk[k] = 0.0;
  // SM 2 state: a conservative score threshold per D-layout candidate row
  // (position 16 rb + 4 grp + i of this lane's rows): the score of the row's
  // running K-th key, -inf until K candidates are in (a candidate scoring
  // below it can never enter the top-K; equal scores go on to the exact key
  // comparison of the merge); the rows' buffer fills live in LDS (cnt_s)
  int nbuf = 0;
  Key thr = 0.0;
  constexpr int RBD = SM == 2 ? RB : 1;
  float thr_d[RBD][4];
  // the row's buffer fill (the same in the group's 16 lanes): in registers
  // for one row block per wave, in LDS (cnt_s) when a lane holds 16 rows
  constexpr bool CREG = RBD == 1;
  int cnt_d[CREG ? RBD : 1][4];
#pragma unroll
  for (int rb = 0; rb < RBD; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      thr_d[rb][i] = NEG_INF;
      if constexpr (CREG) cnt_d[rb][i] = 0;
    }
  if constexpr (SM == 2 && !CREG) {
    if (lane < PW) cnt_s[w][lane] = 0;
    wave_lds_sync();
  }
  // the wave's positions span fewer than S: chunks below the first one's
  // distant count are distant for all of them
  const int nd_lo = pw0 < N ? n_distant(pw0, W, S) : 0;
  // SM 1 state: lane p owns position pw0 + p outright: its buffer fill and
  // its score threshold (the running K-th key's score, -inf until K are in)
  int cnt1 = 0;
  float thr1 = NEG_INF;
  // SM 1: merge every lane's buffer (at most 16) into its list
  auto flush1 = [&]() __attribute__((always_inline)) {
    wave_lds_sync();
    Key nk[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const Key x = sel_key(cbs_s[w][j][lane], cbc_s[w][j][lane]);
      nk[j] = j < cnt1 ? x : 0.0;
    }
    bitonic_sort_desc<16>(nk);
    merge_top<KC>(tk, nk);
    Key th = tk[KC - 1];
    if (K < KC) {
#pragma unroll
      for (int k = 0; k < KC; ++k) th = k == K - 1 ? tk[k] : th;
    }
    thr1 = th == 0.0 ? NEG_INF : key_score(th);
    cnt1 = 0;
    wave_lds_sync();
  };
  // merge every owner lane's buffered candidates into its top-K, 16 at a time
  // (bitonic sort of the 16, then a bitonic merge into the list); the lanes
  // of the wave take part together
  auto flush = [&]() __attribute__((always_inline)) {
    if constexpr (SM == 2 && CREG) {
      if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) cnt_s[w][4 * grp + i] = cnt_d[0][i];
      }
    }
    wave_lds_sync();
    if constexpr (SM == 2) nbuf = lane < PW ? cnt_s[w][lane] : 0;
#pragma unroll
    for (int g16 = 0; g16 < SELBUF; g16 += 16) {
      if (__ballot(lane < PW && nbuf > g16) == 0) break;
      Key nk[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int pl = lane < PW ? lane : 0;
        const Key x = sel_key(cbs_s[w][g16 + j][pl], cbc_s[w][g16 + j][pl]);
        nk[j] = g16 + j < nbuf ? x : 0.0;
      }
      bitonic_sort_desc<16>(nk);
      merge_top<KC>(tk, nk);
    }
    thr = tk[KC - 1];
    if (K < KC) {
#pragma unroll
      for (int k = 0; k < KC; ++k) thr = k == K - 1 ? tk[k] : thr;
    }
    nbuf = 0;
    if constexpr (SM == 2) {
      if (lane < PW) {
        thr_s[w][lane] = thr == 0.0 ? NEG_INF : key_score(thr);
        cnt_s[w][lane] = 0;
      }
      wave_lds_sync();
#pragma unroll
      for (int rb = 0; rb < RBD; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          thr_d[rb][i] = thr_s[w][16 * rb + 4 * grp + i];
          if constexpr (CREG) cnt_d[rb][i] = 0;
        }
      wave_lds_sync();
    }
  };
  const int nd_w = (pw0 < N) ? n_distant(min(pw0 + PW - 1, N - 1), W, S) : 0;
  const int nd_wg = n_distant(min(tile * PWG + PWG - 1, N - 1), W, S);
  const T* kLg = kL + (size_t)bg * C * DH;
  const T* eg = e + (size_t)bg * C;

  typedef typename Frag<T>::type VT;
  VT pre[NV > 0 ? NV : 1];
  float pre_e = 0.f;
  u16x8 preh[URN], prel[URN];  // kL' tile vectors (u path)
  auto fetch = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int el = (tid * NV + v) * VEC;
      const int row = el / DH, cc = el - row * DH;
      const int c = min(t0 + row, C - 1);
      if constexpr (sizeof(T) == 2) {
        pre[v] = *reinterpret_cast<const VT*>(kLg + (size_t)c * DH + cc);
      } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(kLg + (size_t)c * DH + cc);
        VT r;
        r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
        pre[v] = r;
      }
    }
    if (tid < RT_TC) pre_e = to_f<T>(eg[min(t0 + tid, C - 1)]);
    if constexpr (UR > 0) {
#pragma unroll
      for (int v = 0; v < UR; ++v) {
        const int el = (tid * UR + v) * 8;
        const int row = el / RR, cc = el - row * RR;
        const size_t o = ((size_t)bg * C + min(t0 + row, C - 1)) * RR + cc;
        preh[v] = *reinterpret_cast<const u16x8*>(klh + o);
        prel[v] = *reinterpret_cast<const u16x8*>(kll + o);
      }
    }
  };
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int el = (tid * NV + v) * VEC;
      const int row = el / DH, cc = el - row * DH;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<VT*>(kl_s + row * KP + cc) = pre[v];
      } else {
        f32x4 a;
        a[0] = pre[v][0]; a[1] = pre[v][1]; a[2] = pre[v][2]; a[3] = pre[v][3];
        *reinterpret_cast<f32x4*>(kl_s + row * KP + cc) = a;
      }
    }
    if (tid < RT_TC) e_s[tid] = pre_e;
    if constexpr (UR > 0) {
#pragma unroll
      for (int v = 0; v < UR; ++v) {
        const int el = (tid * UR + v) * 8;
        const int row = el / RR, cc = el - row * RR;
        *reinterpret_cast<u16x8*>(klh_s + row * RP + cc) = preh[v];
        *reinterpret_cast<u16x8*>(kll_s + row * RP + cc) = prel[v];
      }
    }
  };

  if (nd_wg > 0) fetch(0);
  for (int t0 = 0; t0 < nd_wg; t0 += RT_TC) {
    __syncthreads();  // previous tile fully consumed
    store();
    __syncthreads();
    if (t0 + RT_TC < nd_wg) fetch(t0 + RT_TC);
    const int c_end = min(t0 + RT_TC, nd_w);
    for (int c0 = t0; c0 < c_end; c0 += 16) {
      FT bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bf[ks] = *reinterpret_cast<const FT*>(kl_s + (c0 + col - t0) * KP + 8 * grp + 32 * ks);
      const float ev = e_s[c0 + col - t0];
      FT kh[URN], kq[URN];
      if constexpr (UR > 0) {
#pragma unroll
        for (int kr = 0; kr < UR; ++kr) {
          const int o = (c0 + col - t0) * RP + 8 * grp + 32 * kr;
          kh[kr] = *reinterpret_cast<const FT*>(klh_s + o);
          kq[kr] = *reinterpret_cast<const FT*>(kll_s + o);
        }
      }
      if constexpr (SM == 1) {
        // scores transposed (landmark keys as the A operand): lane (grp, col)
        // holds chunks c0 + 4 grp + i of position 16 rb + col, turned around
        // through LDS so that lane p holds all 16 chunks of position p
        const f32x4 ev4 = *reinterpret_cast<const f32x4*>(&e_s[c0 - t0 + 4 * grp]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc = mma16(bf[ks], ahi[rb][0][ks], acc);
            if constexpr (HAS_LO) acc = mma16(bf[ks], alo[rb][0][ks], acc);
          }
          if constexpr (UR > 0) {
#pragma unroll
            for (int kr = 0; kr < UR; ++kr) {
              acc = mma16(kh[kr], uhi[rb][kr], acc);
              acc = mma16(kq[kr], uhi[rb][kr], acc);
              acc = mma16(kh[kr], ulo[rb][kr], acc);
            }
          }
          f32x4 sv;
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = fmaf(acc[i], scale, ev4[i]);
          *reinterpret_cast<f32x4*>(&sc_s[w][16 * rb + col][4 * grp]) = sv;
        }
        wave_lds_sync();
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; j += 4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(&sc_s[w][lane][j]);
          v[j] = x[0]; v[j + 1] = x[1]; v[j + 2] = x[2]; v[j + 3] = x[3];
        }
        if (c0 + 15 >= nd_lo) {
          // chunks that are not distant for this position never pass (NaN
          // compares false, also against a threshold of -inf)
          const int lim = mynd - c0;
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = j < lim ? v[j] : __builtin_nanf("");
        }
        // append the candidates that reach the position's threshold; a full
        // buffer is merged first (the rest of the step is then filtered
        // against the refreshed threshold)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          bool p = v[j] >= thr1;
          if (__ballot(p) == 0) continue;
          if (__ballot(p && cnt1 == SB) != 0) {
            flush1();
            p = v[j] >= thr1;
          }
          if (p) {
            cbs_s[w][cnt1][lane] = v[j];
            cbc_s[w][cnt1][lane] = c0 + j;
          }
          cnt1 += p ? 1 : 0;
        }
        continue;
      }
      float sv_d[RBD][4];  // SM 2: this step's scores of the lane's candidate rows
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 best;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            acc = mma16(ahi[rb][hh][ks], bf[ks], acc);
            if constexpr (HAS_LO) acc = mma16(alo[rb][hh][ks], bf[ks], acc);
          }
          if constexpr (UR > 0) {
#pragma unroll
            for (int kr = 0; kr < UR; ++kr) {
              acc = mma16(uhi[rb][kr], kh[kr], acc);
              acc = mma16(uhi[rb][kr], kq[kr], acc);
              acc = mma16(ulo[rb][kr], kh[kr], acc);
            }
          }
          if (hh == 0)
            best = acc;
          else
#pragma unroll
            for (int i = 0; i < 4; ++i) best[i] = fmaxf(best[i], acc[i]);
        }
        // D layout: position 16 rb + 4 grp + i, chunk c0 + col
        if constexpr (SM == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sv_d[rb][i] = fmaf(best[i], scale, ev);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) sc_s[w][16 * rb + 4 * grp + i][col] = fmaf(best[i], scale, ev);
        }
      }
      if constexpr (SM == 2) {
        // filter in place: candidates scoring at least their row's threshold
        // go to the row's buffer, ranked among the group's 16 lanes (one per
        // chunk of the step); most steps keep none and end at one ballot
        const int c = c0 + col;
        const bool edge = c0 + 15 >= nd_lo;  // some chunk may not be distant for some row
        bool pass[RBD][4];
        bool anyp = false;
#pragma unroll
        for (int rb = 0; rb < RBD; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pass[rb][i] = sv_d[rb][i] >= thr_d[rb][i];
            if (edge) {
              const int pp = pw0 + 16 * rb + 4 * grp + i;
              pass[rb][i] = pass[rb][i] && pp < N && c < n_distant(pp, W, S);
            }
            anyp |= pass[rb][i];
          }
        if (__ballot(anyp) == 0) continue;
        bool full = false;
#pragma unroll
        for (int rb = 0; rb < RBD; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint64_t bm = __ballot(pass[rb][i]);
            if (bm == 0) continue;
            const uint32_t gm = (uint32_t)(bm >> (16 * grp)) & 0xFFFFu;
            const int pr = 16 * rb + 4 * grp + i;
            int base;
            if constexpr (CREG) base = cnt_d[rb][i];
            else base = cnt_s[w][pr];
            if (pass[rb][i]) {
              const int slot = base + __popc(gm & ((1u << col) - 1u));
              cbs_s[w][slot][pr] = sv_d[rb][i];
              cbc_s[w][slot][pr] = c;
            }
            const int nc = base + __popc(gm);
            if constexpr (CREG) cnt_d[rb][i] = nc;
            else if (col == 0) cnt_s[w][pr] = nc;
            full |= nc > SELBUF - 16;
          }
        if (__ballot(full) != 0) flush();
        continue;
      }
      wave_lds_sync();
      if constexpr (SM == 0) {
        if (lane < PW) {
          float v[16];
#pragma unroll
          for (int j = 0; j < 16; j += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(&sc_s[w][lane][j]);
            v[j] = x[0]; v[j + 1] = x[1]; v[j + 2] = x[2]; v[j + 3] = x[3];
          }
          Key nk[16];
          bool any = false;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            // masked arithmetically (a select here became a branch per
            // candidate): absent candidates get key 0, below every real one
            nk[j] = sel_key(v[j], c0 + j) * (double)(c0 + j < mynd);
            any |= nk[j] > thr;
          }
          if (__ballot(any) != 0) {
            bitonic_sort_desc<16>(nk);
            merge_top<KC>(tk, nk);
            thr = tk[KC - 1];
            if (K < KC) {
#pragma unroll
              for (int k = 0; k < KC; ++k) thr = k == K - 1 ? tk[k] : thr;
            }
          }
        }
        wave_lds_sync();
        continue;
      }
    }
  }

  if constexpr (SM == 1) {
    if (__ballot(cnt1 > 0) != 0) flush1();
  }
  if constexpr (SM == 2) {
    bool any = false;
    if constexpr (CREG) {
#pragma unroll
      for (int i = 0; i < 4; ++i) any |= cnt_d[0][i] > 0;
    } else {
      wave_lds_sync();
      any = lane < PW && cnt_s[w][lane] > 0;
    }
    if (__ballot(any) != 0) flush();
  }

  // output: indices ascending, -1 padded; per-head fp32 scores of the selected chunks
  if (lane < PW && mypos < N) {
    // sort the K best by chunk id (insertion sort over a small register array)
    int ids[KC];
    float sv[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      ids[k] = (k < K && tk[k] != 0.0) ? key_chunk(tk[k]) : 0x7FFFFFFF;
      sv[k] = key_score(tk[k]);
    }
#pragma unroll
    for (int a = 0; a < KC; ++a)
#pragma unroll
      for (int bb = KC - 1; bb > a; --bb) {
        const bool sw = ids[bb] < ids[bb - 1];
        const int ti = ids[bb];
        const float ts = sv[bb];
        ids[bb] = sw ? ids[bb - 1] : ti;
        sv[bb] = sw ? sv[bb - 1] : ts;
        ids[bb - 1] = sw ? ti : ids[bb - 1];
        sv[bb - 1] = sw ? ts : sv[bb - 1];
      }
    int32_t* dst = topk_idx + ((size_t)bg * N + mypos) * K;
    // a lane's row of K ids is contiguous: 16-byte stores where K and the
    // pointer allow it (uniform over the wave)
    const bool v4i = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0;
    if (v4i) {
#pragma unroll
      for (int k = 0; k < KC; k += 4)
        if (k < K) {
          int4 v;
          v.x = ids[k] == 0x7FFFFFFF ? -1 : ids[k];
          v.y = ids[k + 1] == 0x7FFFFFFF ? -1 : ids[k + 1];
          v.z = ids[k + 2] == 0x7FFFFFFF ? -1 : ids[k + 2];
          v.w = ids[k + 3] == 0x7FFFFFFF ? -1 : ids[k + 3];
          *reinterpret_cast<int4*>(dst + k) = v;
        }
    } else {
#pragma unroll
      for (int k = 0; k < KC; ++k)
        if (k < K) dst[k] = ids[k] == 0x7FFFFFFF ? -1 : ids[k];
    }
    if constexpr (G >= 2) {
      // the per-head scores below read every position's ids from LDS,
      // position-major ([p][k], K <= SELBUF) in the buffer's space
      int* ids_s = &cbc_s[w][0][0];
#pragma unroll
      for (int k = 0; k < KC; ++k)
        if (k < K) ids_s[lane * SELBUF + k] = ids[k] == 0x7FFFFFFF ? -1 : ids[k];
    }
    if (G == 1 && topk_score != nullptr) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float* ds = topk_score + (((size_t)b * Hq + g * G + hh) * N + mypos) * K;
        // log-sum-exp of the head's selected scores (-inf when none is valid)
        float lm = NEG_INF, ls = 0.f;
        auto lse_add = [&](float x) __attribute__((always_inline)) {
          const float mn = fmaxf(lm, x);
          ls = ls * __expf(lm - mn) + __expf(x - mn);
          lm = mn;
        };
        if constexpr (G == 1) {
          float so[KC];
#pragma unroll
          for (int k = 0; k < KC; ++k) {
            const bool ok = k < K && ids[k] != 0x7FFFFFFF;
            so[k] = ok ? sv[k] : __builtin_nanf("");
            if (ok) lse_add(sv[k]);
          }
          if (v4i && (reinterpret_cast<uintptr_t>(topk_score) & 15) == 0) {
#pragma unroll
            for (int k = 0; k < KC; k += 4)
              if (k < K) *reinterpret_cast<f32x4*>(ds + k) = f32x4{so[k], so[k + 1], so[k + 2], so[k + 3]};
          } else {
#pragma unroll
            for (int k = 0; k < KC; ++k)
              if (k < K) ds[k] = so[k];
          }
        }
        // grouped heads: their per-head scores follow below
        if (sel_lse != nullptr)
          sel_lse[((size_t)b * Hq + g * G + hh) * N + mypos] = lm == NEG_INF ? NEG_INF : lm + __logf(ls);
      }
    }
  }

  // Grouped heads: each head's fp32 score of every selected chunk (NaN in
  // empty slots) and the log-sum-exp of a head's selected scores (the
  // selection ran on the group maximum). The scoring fragments of all the
  // wave's positions and heads are still in registers: per position, one MFMA
  // product per head of that position's 16 selected landmark rows (A,
  // gathered from L2, the next block's rows in flight) against the 16
  // positions' queries (B, the scan's fragments), of which the position's own
  // column of D is kept: lane (grp, r) holds its slots 4 grp .. 4 grp + 3, a
  // 16-byte run of the scores, and the log-sum-exp combines the four lanes.
  if constexpr (G >= 2) {
    if (topk_score != nullptr || sel_lse != nullptr) {
      wave_lds_sync();
      constexpr int NKB = (KC + 15) / 16;
      const int* ids_s = &cbc_s[w][0][0];
      const int np = min(PW, N - pw0);  // positions of this wave (uniform; <= 0 past the end)
      // a lane's four slots are one 16-byte run where K and the pointer allow
      const bool sc_v4 = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(topk_score) & 15) == 0;
      struct BIn {
        FT kf[KS];
        int c4[4];    // ids of slots 16 kb + 4 grp + i
        float ev4[4]; // and their biases
      };
      auto fetchb = [&](BIn& x, int p, int kb) __attribute__((always_inline)) {
        const int pp = p < np ? p : 0;
        const int slot = 16 * kb + col;
        const int c = (slot < K && p < np) ? ids_s[pp * SELBUF + slot] : -1;
        const T* kr = kLg + (size_t)(c >= 0 ? c : 0) * DH + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x.kf[ks] = ld8<T>(kr + 32 * ks);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s4 = 16 * kb + 4 * grp + i;
          const int ci = (s4 < K && p < np) ? ids_s[pp * SELBUF + s4] : -1;
          x.c4[i] = ci;
          x.ev4[i] = to_f<T>(eg[ci >= 0 ? ci : 0]);
        }
      };
      BIn bcur, bnxt;
      if (np > 0) fetchb(bcur, 0, 0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        for (int r = 0; r < 16; ++r) {
          const int p = 16 * rb + r;
          if (p >= np) break;  // uniform
          const int pos = pw0 + p;
          const bool mine = col == r;
          float lm2[G], ls2[G];
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            lm2[hh] = NEG_INF;
            ls2[hh] = 0.f;
          }
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            // the next (position, block)'s rows in flight
            if (kb + 1 < NKB) fetchb(bnxt, p, kb + 1);
            else fetchb(bnxt, p + 1, 0);
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
              f32x4 acc = zero4();
#pragma unroll
              for (int ks = 0; ks < KS; ++ks) {
                acc = mma16(bcur.kf[ks], ahi[rb][hh][ks], acc);
                if constexpr (HAS_LO) acc = mma16(bcur.kf[ks], alo[rb][hh][ks], acc);
              }
              // D layout: slot 16 kb + 4 grp + i, position 16 rb + col
              f32x4 sc;
              float mx = NEG_INF;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                sc[i] = bcur.c4[i] >= 0 ? fmaf(acc[i], scale, bcur.ev4[i]) : __builtin_nanf("");
                if (bcur.c4[i] >= 0) mx = fmaxf(mx, sc[i]);
              }
              if (mine && topk_score != nullptr) {
                float* dsc = topk_score + (((size_t)b * Hq + g * G + hh) * N + pos) * K;
                const int s0 = 16 * kb + 4 * grp;
                if (sc_v4) {
                  if (s0 < K) *reinterpret_cast<f32x4*>(dsc + s0) = sc;
                } else {
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    if (s0 + i < K) dsc[s0 + i] = sc[i];
                }
              }
              // the position's four lanes (grp = 0..3, same col) combine
              mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
              mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
              const float mn = fmaxf(lm2[hh], mx);
              float ex = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                ex += (bcur.c4[i] >= 0 && mn != NEG_INF) ? __expf(sc[i] - mn) : 0.f;
              ex += __shfl_xor(ex, 16, 64);
              ex += __shfl_xor(ex, 32, 64);
              ls2[hh] = (lm2[hh] == NEG_INF ? 0.f : ls2[hh] * __expf(lm2[hh] - mn)) + ex;
              lm2[hh] = mn;
            }
            bcur = bnxt;
          }
          if (mine && grp == 0 && sel_lse != nullptr) {
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
              sel_lse[((size_t)b * Hq + g * G + hh) * N + pos] =
                  lm2[hh] == NEG_INF ? NEG_INF : lm2[hh] + __logf(ls2[hh]);
          }
        }
      }
    }
  }
}

template <typename T, typename QT, int G, int DH, int KC, int UR>
static hipError_t route_go(const Dims& p, const void* qs, const void* kL, const void* e,
                           int32_t* idx, float* sc, float* sl, const RouteU& ru, hipStream_t st) {
  constexpr int PWG = 4 * 16 * (G >= 4 ? 1 : 4 / G);
  const int ntiles = (p.N + PWG - 1) / PWG;
  // one head per KV head: buffer the candidates only when the scan is long
  // (with a few hundred chunks most candidates fill the lists anyway)
  auto kern = (G == 1 && p.C < 512) ? k_route<T, QT, G, DH, KC, UR, false>
                                    : k_route<T, QT, G, DH, KC, UR, true>;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), 0, st, (const QT*)qs,
                     (const T*)kL, (const T*)e, idx, sc, sl, p.N, p.C, p.Hkv, p.K, p.W, p.S, p.scale,
                     ntiles, ru.u, ru.klh, ru.kll);
  return hipGetLastError();
}

template <typename T, typename QT, int G, int DH, int UR>
static hipError_t route_k(const Dims& p, const void* qs, const void* kL, const void* e,
                          int32_t* idx, float* sc, float* sl, const RouteU& ru, hipStream_t st) {
  if (p.K <= 4) return route_go<T, QT, G, DH, 4, UR>(p, qs, kL, e, idx, sc, sl, ru, st);
  if (p.K <= 8) return route_go<T, QT, G, DH, 8, UR>(p, qs, kL, e, idx, sc, sl, ru, st);
  if (p.K <= 16) return route_go<T, QT, G, DH, 16, UR>(p, qs, kL, e, idx, sc, sl, ru, st);
  if constexpr (UR > 0) return hipErrorInvalidValue;  // the u path serves K <= 16
  else return route_go<T, QT, G, DH, 32, UR>(p, qs, kL, e, idx, sc, sl, ru, st);
}

template <typename T, typename QT, int G>
static hipError_t route_d(const Dims& p, const void* qs, const void* kL, const void* e, int32_t* idx,
                          float* sc, float* sl, const RouteU& ru, hipStream_t st) {
  if constexpr (G == 1 && sizeof(T) == 2 && sizeof(QT) == 2) {
    if (ru.u != nullptr) {
      if (p.d == 64)
        return p.r == 32 ? route_k<T, QT, G, 64, 1>(p, qs, kL, e, idx, sc, sl, ru, st)
                         : route_k<T, QT, G, 64, 2>(p, qs, kL, e, idx, sc, sl, ru, st);
      return p.r == 32 ? route_k<T, QT, G, 128, 1>(p, qs, kL, e, idx, sc, sl, ru, st)
                       : route_k<T, QT, G, 128, 2>(p, qs, kL, e, idx, sc, sl, ru, st);
    }
  }
  if (p.d == 64) return route_k<T, QT, G, 64, 0>(p, qs, kL, e, idx, sc, sl, ru, st);
  return route_k<T, QT, G, 128, 0>(p, qs, kL, e, idx, sc, sl, ru, st);
}

template <typename T, typename QT>
static hipError_t route_g(const Dims& p, const void* qs, const void* kL, const void* e, int32_t* idx,
                          float* sc, float* sl, const RouteU& ru, hipStream_t st) {
  switch (p.G) {
    case 1: return route_d<T, QT, 1>(p, qs, kL, e, idx, sc, sl, ru, st);
    case 2: return route_d<T, QT, 2>(p, qs, kL, e, idx, sc, sl, ru, st);
    case 4: return route_d<T, QT, 4>(p, qs, kL, e, idx, sc, sl, ru, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_route(const Dims& p, const void* qs, bool q_is_f32, const void* kL, const void* e,
                        int32_t* topk_idx, float* topk_score, float* sel_lse, hipStream_t st,
                        const RouteU& ru) {
  if (ru.u != nullptr && !route_u_ok(p)) return hipErrorInvalidValue;
  if (p.C > (1 << 20)) return hipErrorInvalidValue;  // selection keys hold 20-bit chunk ids
  if (p.dtype == 1) {
    if (q_is_f32) return route_g<uint16_t, float>(p, qs, kL, e, topk_idx, topk_score, sel_lse, ru, st);
    return route_g<uint16_t, uint16_t>(p, qs, kL, e, topk_idx, topk_score, sel_lse, ru, st);
  }
  return route_g<float, float>(p, qs, kL, e, topk_idx, topk_score, sel_lse, ru, st);
}

bool route_u_ok(const Dims& p) {
  // K <= 16: with 32 selection keys per lane on top of the u operands the
  // kernel would spill (the q_hat path then serves K up to 32)
  return p.dtype == 1 && p.G == 1 && (p.r == 32 || p.r == 64) && p.K <= 16;
}

// W_up[h]^T kL_c for every (b, query head, chunk): the Q-Cal part of the
// surrogate score moved onto the landmark side, as bf16 hi + lo planes
// [B, Hq, C, r] (fp32 sums of exact bf16 products). One workgroup per
// (b, head, 2048 / r chunks): W_up[h] and the chunks' landmark rows are
// staged in LDS with coalesced loads, r / 8 lanes share a chunk and each
// computes 8 of its r outputs.
template <int DH>
__global__ __launch_bounds__(256) void k_route_klp(const uint16_t* __restrict__ W_up,
                                                   const uint16_t* __restrict__ kL,
                                                   uint16_t* __restrict__ klh,
                                                   uint16_t* __restrict__ kll, int Hq, int Hkv,
                                                   int C, int r) {
  __shared__ float wu[DH * 64];            // W_up[h] [DH][r], r <= 64
  __shared__ float kt[64 * (DH + 1)];      // landmark rows of the block's chunks
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, b = bh / Hq, h = bh - b * Hq, g = h / (Hq / Hkv);
  const int cpb = 2048 / r, c0 = blockIdx.x * cpb;
  for (int x = tid; x < DH * r; x += 256) wu[x] = bf2f(W_up[(size_t)h * DH * r + x]);
  const uint16_t* kg = kL + ((size_t)b * Hkv + g) * C * DH;
  for (int x = tid; x < cpb * DH; x += 256) {
    const int cl = x / DH, dd = x - cl * DH;
    kt[cl * (DH + 1) + dd] = bf2f(kg[(size_t)min(c0 + cl, C - 1) * DH + dd]);
  }
  __syncthreads();
  const int lpc = r / 8, cl = tid / lpc, j0 = (tid - cl * lpc) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float* kr = kt + cl * (DH + 1);
#pragma unroll 8
  for (int dd = 0; dd < DH; ++dd) {
    const float kv = kr[dd];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[jj] = fmaf(kv, wu[dd * r + j0 + jj], acc[jj]);
  }
  const int c = c0 + cl;
  if (c < C) {
    const size_t o = (((size_t)b * Hq + h) * C + c) * r + j0;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const uint16_t hi = f2bf(acc[jj]);
      klh[o + jj] = hi;
      kll[o + jj] = f2bf(acc[jj] - bf2f(hi));
    }
  }
}

hipError_t launch_route_klp(const Dims& p, const void* W_up, const void* kL, uint16_t* klh,
                            uint16_t* kll, hipStream_t st) {
  if ((long)p.B * p.Hq * p.C * p.r == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.C + 2048 / p.r - 1) / (2048 / p.r)), (unsigned)(p.B * p.Hq));
  if (p.d == 64)
    hipLaunchKernelGGL(k_route_klp<64>, grid, dim3(256), 0, st, (const uint16_t*)W_up,
                       (const uint16_t*)kL, klh, kll, p.Hq, p.Hkv, p.C, p.r);
  else
    hipLaunchKernelGGL(k_route_klp<128>, grid, dim3(256), 0, st, (const uint16_t*)W_up,
                       (const uint16_t*)kL, klh, kll, p.Hq, p.Hkv, p.C, p.r);
  return hipGetLastError();
}

}  // namespace hils
