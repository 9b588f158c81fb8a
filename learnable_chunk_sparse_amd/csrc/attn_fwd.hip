// HiLS prefill forward: sliding-window attention, attention inside each
// selected chunk, and the hierarchical fusion, in one kernel per query tile.
//
// Paper: Fig. 3 (inter-chunk softmax gives each chunk its mass, intra-chunk
// softmax spreads it over the chunk's tokens), the engineersofai abstract
// (each query attends to each retrieved chunk independently; the outputs are
// fused by the retrieval scores), "Limitations of Naive Sparse Attention"
// (local sliding window plus top-K distant chunks). For query row (h, i):
//   O_W, lse_W : exact causal softmax attention over the window [n_dist*S, i]
//   O_c, lse_c : exact softmax attention over the S tokens of chunk c in T(i)
//   L = log(sum_{c in T} exp(s_c) + exp(lse_W))
//   o = sum_{c in T} exp(s_c - L) O_c + exp(lse_W - L) O_W
//
// Products use the transposed form S^T = K Q^T (tokens x rows), whose
// accumulator layout is exactly the P^T operand of O^T = V^T P^T once the
// token order inside each 32-token step is permuted identically on both
// operands; V is transposed once per call into a token-permuted copy
// (k_vt_perm).
//
// Shared-block strategy (this file): a tile is 128 rows (128/G positions x G
// heads) of one (batch, KV head); wave w owns rows 32w .. 32w+31 and keeps
// their output accumulators in registers. The tile's work is a list of
// 64-token blocks: its window blocks, then the union of the chunks its rows
// selected (ascending). Each block's K and V^T are staged once into an LDS
// slot (two slots; the next blocks' global loads are in flight in registers
// while the current one is multiplied) and read by all four waves.
//   Window blocks: banded flash attention of each wave's rows (blocks outside
//     a wave's windows are skipped, masks only on edge blocks).
//   After the window: L = log(exp(lse_W) + exp(lse_sel)) with lse_sel the
//     log-sum-exp of the row's selected scores, and the window output is
//     scaled by exp(lse_W - L).
//   Chunk blocks: every row keeps a cursor into its ascending selection list;
//     row blocks where no row selected the chunk are skipped, the others add
//     exp(s_c - L) O_c (rows that did not select it get weight 0).
// With no per-wave accumulator copies the tile needs ~55 KB of LDS (d = 64),
// so two tiles share a CU. Tiles whose selections are spread over many more
// chunks than they select use the bucketed strategy of attn_fwd_sparse.hip.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

// ---------------------------------------------------------------- V^T copy
// vt[bg][d][Np] (Np = N rounded up to 64, zero padded) with the tokens of
// every 32-token group stored in the order 0-3,16-19, 4-7,20-23, 8-11,24-27,
// 12-15,28-31, so that lane group g of an MFMA fragment finds its 8 tokens
// {4g..4g+3, 16+4g..16+4g+3} contiguous at slots 8g..8g+7.
// One workgroup per 64-token block: the block's rows come in as 16-byte
// vectors into an LDS tile, and each output vector (8 consecutive slots of
// one d row) is gathered from the tile's column and written as 16 bytes.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_vt_perm(const T* __restrict__ v, T* __restrict__ vt, int N,
                                                 int Np) {
  constexpr int V = 16 / sizeof(T);      // elements per 16-byte vector
  constexpr int TP = sizeof(T) == 2 ? DH + 2 : DH + 1;  // tile pitch: an odd number of words
  constexpr int NV = 64 * DH / V;                         // vectors per block
  __shared__ __align__(16) T tile[64 * TP];
  const int bg = blockIdx.y, t0 = blockIdx.x * 64;
  const T* src = v + (size_t)bg * N * DH;
  // rows in: vector x = token t, dims dv .. dv + V - 1 (rows past N read as 0)
  T in[NV / 256][V];
#pragma unroll
  for (int i = 0; i < NV / 256; ++i) {
    const int x = threadIdx.x + 256 * i;
    const int t = x / (DH / V), dv = (x - t * (DH / V)) * V;
    const bool ok = t0 + t < N;
    const T* p = src + (size_t)(ok ? t0 + t : 0) * DH + dv;
    if constexpr (sizeof(T) == 2) {
      const u16x8 a = *reinterpret_cast<const u16x8*>(p);
#pragma unroll
      for (int j = 0; j < 8; ++j) in[i][j] = ok ? a[j] : (T)0;
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
      for (int j = 0; j < 4; ++j) in[i][j] = ok ? a[j] : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < NV / 256; ++i) {
    const int x = threadIdx.x + 256 * i;
    const int t = x / (DH / V), dv = (x - t * (DH / V)) * V;
#pragma unroll
    for (int j = 0; j < V; ++j) tile[t * TP + dv + j] = in[i][j];
  }
  __syncthreads();
  // vectors out: row dd, slots s .. s + V - 1 of the block
  T* dst = vt + (size_t)bg * DH * Np + t0;
#pragma unroll
  for (int i = 0; i < NV / 256; ++i) {
    const int x = threadIdx.x + 256 * i;
    const int dd = x / (64 / V), s0 = (x - dd * (64 / V)) * V;
    T o[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int s = s0 + j;  // storage slot within the 64-token block
      const int half = s >> 5, sl = s & 31;
      const int g8 = sl >> 3, e = sl & 7;
      const int t = 32 * half + (e < 4 ? 4 * g8 + e : 16 + 4 * g8 + (e - 4));
      o[j] = tile[t * TP + dd];
    }
    if constexpr (sizeof(T) == 2) {
      u16x8 w;
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = o[j];
      *reinterpret_cast<u16x8*>(dst + (size_t)dd * Np + s0) = w;
    } else {
      *reinterpret_cast<f32x4*>(dst + (size_t)dd * Np + s0) = f32x4{o[0], o[1], o[2], o[3]};
    }
  }
}

template __global__ void k_vt_perm<uint16_t, 64>(const uint16_t*, uint16_t*, int, int);
template __global__ void k_vt_perm<uint16_t, 128>(const uint16_t*, uint16_t*, int, int);
template __global__ void k_vt_perm<float, 64>(const float*, float*, int, int);
template __global__ void k_vt_perm<float, 128>(const float*, float*, int, int);

// LDS slot holding one 64-token block: K rows and V^T rows (token-permuted),
// pitches padded by 16 bytes so the 16-byte fragment reads of 16 lanes hit
// distinct banks.
template <typename T, int DH>
struct Slot {
  static constexpr int VE = 16 / (int)sizeof(T);         // elements per 16-byte vector
  static constexpr int KP = DH + VE;                      // K row pitch
  static constexpr int VP = 64 + VE;                      // V^T row pitch
  static constexpr int KE = 64 * KP;                      // K part (elements)
  static constexpr int ELEMS = KE + DH * VP;
  static constexpr int KV = 64 * DH / VE;                 // 16-byte vectors of K
  static constexpr int VPT = 2 * KV / 256;                // vectors per thread (K then V^T)
};

template <typename T, int G, int DH>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && DH == 64) ? 2 : 1) void k_attn_fwd(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_score,
    const float* __restrict__ sel_lse, T* __restrict__ o, float* __restrict__ lse, int N, int Np,
    int Hkv, int K, int W, int S, float scale, int ntiles, int C) {
  typedef typename Frag<T>::type FT;
  typedef Slot<T, DH> SG;
  constexpr int R = 128;      // rows per tile: 2 row blocks of 16 per wave
  constexpr int TP = R / G;   // positions per tile
  constexpr int KS = DH / 32;
  constexpr int MB = DH / 16;
  constexpr bool FIXREF = DH == 64;  // chunk softmax against the window maximum

  extern __shared__ __align__(16) unsigned char smem[];
  T* slots = reinterpret_cast<T*>(smem);                             // [2][ELEMS]
  const int K1 = K + 1;  // selection lists end with a sentinel (-1 / 0)
  int* tkc = reinterpret_cast<int*>(slots + 2 * SG::ELEMS);          // [TP][K + 1] selected chunks
  float* tks = reinterpret_cast<float*>(tkc + TP * K1);             // [R][K + 1] their scores
  int* flg = reinterpret_cast<int*>(tks + R * K1);                  // [C + 1] union flags / offsets
  int* ulist = flg + C + 1;                                         // [min(C, TP K)] union, ascending
  __shared__ int wsum[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gl = lane >> 4, cl = lane & 15;
  int tx, bg;
  xcd_block(tx, bg);
  const int tile = ntiles - 1 - tx;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * TP;
  const int plast = min(p0 + TP - 1, N - 1);
  const int ndmax = n_distant(plast, W, S);
  // K and V^T of this (batch, KV head) through buffer resources: K rows past
  // N read as zero (they are masked), V^T is padded to Np
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bg * N * DH, N * DH * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vt + (size_t)bg * DH * Np, DH * Np * (int)sizeof(T));

  // ------------------------------------------------ per-lane rows
  // wave w owns rows 32 w + 16 cb + cl, cb = 0, 1 (all four lanes of a
  // column hold the same row)
  FT qf[2][KS];
  int prow[2], wsr[2], cbase[2], sbase[2], cur[2];
  // global row index (b, head, position) of row block cb (recomputed where
  // needed rather than held across the item loop)
  auto row_off = [&](int cb) __attribute__((always_inline)) -> size_t {
    const int r = 32 * w + 16 * cb + cl;
    const int pos = min(p0 + r / G, N - 1);
    return ((size_t)b * Hq + g * G + r % G) * N + pos;
  };
  float lsel[2], Lr[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = 32 * w + 16 * cb + cl;
    const int pos = p0 + r / G, hh = r % G;
    cbase[cb] = (r / G) * K1;
    sbase[cb] = r * K1;
    prow[cb] = pos < N ? pos : -1;
    wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
    const int pc = pos < N ? pos : N - 1;
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pc;
    lsel[cb] = sel_lse[ro];
    cur[cb] = 0;
    const T* src = q + ro * DH + 8 * gl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = ld8<T>(src + 32 * ks);
  }
  // rows of this wave: positions pw_lo .. pw_hi; masks are needed on blocks
  // that are not strictly inside every row's window
  const int pw_lo = p0 + 32 * w / G;
  const int pw_hi = min(p0 + (32 * w + 31) / G, N - 1);
  const bool wave_live = pw_lo < N;
  const bool all_valid = p0 + (32 * w + 31) / G < N;
  const int ws_lo = wave_live ? n_distant(pw_lo, W, S) * S : 0;
  const int ws_hi = wave_live ? n_distant(pw_hi, W, S) * S : 0;

  // m: the row's reference (log2 units) that probabilities are taken
  // against, -inf until the row's first scores; cneg = -m in every element,
  // the initial accumulator of the chunk score products
  float m[2], lsum[2];
  f32x4 oacc[MB][2], cneg[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    m[cb] = NEG_INF;
    lsum[cb] = 0.f;
    cneg[cb] = zero4();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] = zero4();
  }
  const float sc2 = scale * LOG2E;

  // ------------------------------------------------ work items
  // items 0 .. nW-1: window blocks kv_lo + 64 n; then the NU union chunks.
  // Block staging: thread vectors s < VPT/2 are K (token, 16-byte part), the
  // rest V^T (dim, part); two blocks are in flight in registers.
  const int kv_lo = n_distant(p0, W, S) * S;
  const int nW = (plast - kv_lo) / 64 + 1;
  u32x4 stg[2][SG::VPT];
  auto issue_kv = [&](u32x4 (&rg)[SG::VPT], int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < SG::VPT; ++s) {
      const int vi = tid + 256 * s;
      if (s < SG::VPT / 2) {
        const int tok = vi / (DH / SG::VE), part = vi - tok * (DH / SG::VE);
        rg[s] = buf_ld16(krs, ((kv0 + tok) * DH + part * SG::VE) * (int)sizeof(T));
      } else {
        const int vj = vi - SG::KV;
        const int dd = vj / (64 / SG::VE), part = vj - dd * (64 / SG::VE);
        rg[s] = buf_ld16(vrs, (dd * Np + kv0 + part * SG::VE) * (int)sizeof(T));
      }
    }
  };
  auto commit = [&](const u32x4 (&rg)[SG::VPT], int slot) __attribute__((always_inline)) {
    T* base = slots + slot * SG::ELEMS;
#pragma unroll
    for (int s = 0; s < SG::VPT; ++s) {
      const int vi = tid + 256 * s;
      T* dst;
      if (s < SG::VPT / 2) {
        const int tok = vi / (DH / SG::VE), part = vi - tok * (DH / SG::VE);
        dst = base + tok * SG::KP + part * SG::VE;
      } else {
        const int vj = vi - SG::KV;
        const int dd = vj / (64 / SG::VE), part = vj - dd * (64 / SG::VE);
        dst = base + SG::KE + dd * SG::VP + part * SG::VE;
      }
      *reinterpret_cast<u32x4*>(dst) = rg[s];
    }
  };
  // the first window blocks do not depend on the selections: start them now
  issue_kv(stg[0], kv_lo);
  if (nW > 1) issue_kv(stg[1], kv_lo + 64);

  // ------------------------------------------------ selections of the tile
  for (int x = tid; x <= ndmax; x += 256) flg[x] = 0;
  if (K % 4 == 0 && (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(topk_score) & 15) == 0) {
    // 16-byte vectors, every load issued before any is used (clamped
    // addresses, no per-element branches); at most four per thread (K <= 32)
    // (ids: TP positions; scores: R = TP G rows)
    const int KV4 = K >> 2, nvi = TP * KV4, nvs = R * KV4;
    int4 vi[4];
    f32x4 vs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = tid + 256 * j;
      const int vc = min(v, nvi - 1), rc = vc / KV4, pc = vc - rc * KV4;
      vi[j] = *reinterpret_cast<const int4*>(topk_idx + ((size_t)bg * N + min(p0 + rc, N - 1)) * K + 4 * pc);
      const int ws2 = min(v, nvs - 1), rs = ws2 / KV4, qs2 = ws2 - rs * KV4;
      vs[j] = *reinterpret_cast<const f32x4*>(
          topk_score + (((size_t)b * Hq + g * G + rs % G) * N + min(p0 + rs / G, N - 1)) * K + 4 * qs2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = tid + 256 * j;
      const int r = v / KV4, part = v - r * KV4;
      if (v < nvi) {
        const bool li = p0 + r < N;
        int* dc = tkc + r * K1 + 4 * part;
        dc[0] = li ? vi[j].x : -1;
        dc[1] = li ? vi[j].y : -1;
        dc[2] = li ? vi[j].z : -1;
        dc[3] = li ? vi[j].w : -1;
      }
      if (v < nvs) {
        const bool ls = p0 + r / G < N;
        float* dsc = tks + r * K1 + 4 * part;
        dsc[0] = ls ? vs[j][0] : 0.f;
        dsc[1] = ls ? vs[j][1] : 0.f;
        dsc[2] = ls ? vs[j][2] : 0.f;
        dsc[3] = ls ? vs[j][3] : 0.f;
      }
    }
    for (int x = tid; x < R; x += 256) {
      if (x < TP) tkc[x * K1 + K] = -1;
      tks[x * K1 + K] = 0.f;
    }
  } else {
    for (int x = tid; x < TP * K1; x += 256) {
      const int pl = x / K1, kk = x - pl * K1;
      const int pos = p0 + pl;
      tkc[x] = (pos < N && kk < K) ? topk_idx[((size_t)bg * N + pos) * K + kk] : -1;
    }
    for (int x = tid; x < R * K1; x += 256) {
      const int r = x / K1, kk = x - r * K1;
      const int pos = p0 + r / G;
      tks[x] = (pos < N && kk < K) ? topk_score[(((size_t)b * Hq + g * G + r % G) * N + pos) * K + kk] : 0.f;
    }
  }
  __syncthreads();
  for (int x = tid; x < TP * K1; x += 256) {
    const int c = tkc[x];
    if (c >= 0 && c < ndmax) flg[c] = 1;
  }
  __syncthreads();
  // union of the selected chunks, ascending: flg becomes offsets, ulist the ids
  int NU = 0;
  if (ndmax > 0) {
    NU = block_excl_scan(flg, ndmax, wsum);
    if (tid == 0) flg[ndmax] = NU;
    __syncthreads();
    for (int c = tid; c < ndmax; c += 256)
      if (flg[c + 1] > flg[c]) ulist[flg[c]] = c;
  }

  const int NIT = nW + NU;
  auto issue = [&](u32x4 (&rg)[SG::VPT], int n) __attribute__((always_inline)) {
    n = min(n, NIT - 1);
    issue_kv(rg, n < nW ? kv_lo + 64 * n : 64 * ulist[n - nW]);
  };

  // ---- window block: banded flash attention over the wave's rows. The
  // reference m moves only when a block's scores exceed it by more than 16
  // (log2 units), or on a row's first scores; the accumulators are rescaled
  // only then. (Scores stay in the exact fp32 product of q and k here: the
  // window log-sum-exp is an output.)
  auto window_block = [&](const T* sl, int kv0, auto masked) __attribute__((always_inline)) {
    constexpr bool MSK = decltype(masked)::value;
    constexpr float SHIFT_AT = 16.f;
    f32x4 sacc[4][2];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) sacc[tb][cb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FT kf = ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) sacc[tb][cb] = mma16(kf, qf[cb][ks], sacc[tb][cb]);
      }
    }
    float bmx[2];
    bool shift = false;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float bmax = NEG_INF;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[tb][cb][i];
          if constexpr (MSK) {
            const int j = kv0 + 16 * tb + 4 * gl + i;
            x = (j <= prow[cb] && j >= wsr[cb]) ? x : NEG_INF;
            sacc[tb][cb][i] = x;
          }
          bmax = fmaxf(bmax, x);
        }
      // block maximum relative to the reference (0 before the first scores)
      bmx[cb] = col_max4(bmax) * sc2 - (m[cb] == NEG_INF ? 0.f : m[cb]);
      shift |= bmx[cb] > SHIFT_AT || (m[cb] == NEG_INF && bmx[cb] != NEG_INF);
    }
    if (__ballot(shift) != 0) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const bool first = m[cb] == NEG_INF;
        const bool up = bmx[cb] > SHIFT_AT || (first && bmx[cb] != NEG_INF);
        const float dlt = up ? bmx[cb] : 0.f;
        const float alpha = first ? 0.f : fast_exp2(-dlt);
        if (up) m[cb] = (first ? 0.f : m[cb]) + dlt;
        lsum[cb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= alpha;
      }
    }
    FT pf[2][2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float mc = m[cb] == NEG_INF ? 0.f : m[cb];
      float ps = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(sacc[tb][cb][i], sc2, -mc));
          sacc[tb][cb][i] = pv;
          ps += pv;
        }
      lsum[cb] += ps;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) pf[cb][ks] = pk8<T>(sacc[2 * ks][cb], sacc[2 * ks + 1][cb]);
    }
    const T* vb = sl + SG::KE;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const FT vf = ld8<T>(vb + (16 * mb + cl) * SG::VP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) oacc[mb][cb] = mma16(vf, pf[cb][ks], oacc[mb][cb]);
      }
  };

  // ---- fusion normaliser once the window is done: L, and the window weight
  auto fuse = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float ls = col_sum4(lsum[cb]);
      const float lW = (m[cb] + __log2f(ls)) * LN2;
      const float mx = fmaxf(lW, lsel[cb]);
      const bool live = prow[cb] >= 0;
      const float L = live ? mx + __logf(__expf(lW - mx) + __expf(lsel[cb] - mx)) : 0.f;
      const float coef = live ? fast_exp2(m[cb] - L * LOG2E) : 0.f;
      Lr[cb] = L;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= coef;
      // chunk phase: the score products start from -m (in score units), so
      // each probability is exp2 of one product times log2(e)/sqrt(d)
      const float mr = live ? -m[cb] / sc2 : 0.f;
      cneg[cb] = f32x4{mr, mr, mr, mr};
    }
  };

  // ---- exp2(x log2(e)/sqrt(d)) of a 64-token block of shifted scores into
  // P^T operands; returns the row sum of the rounded probabilities (for bf16
  // an MFMA with an all-ones operand, exactly the weights the PV product uses)
  auto chunk_probs = [&](f32x4 (&sacc)[4], FT (&pf)[2]) __attribute__((always_inline)) -> float {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[tb][i] = fast_exp2(sacc[tb][i] * sc2);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pf[ks] = pk8<T>(sacc[2 * ks], sacc[2 * ks + 1]);
    if constexpr (sizeof(T) == 2) {
      f32x4 s4 = mma16(ones_frag(), pf[0], zero4());
      s4 = mma16(ones_frag(), pf[1], s4);
      return s4[0];
    } else {
      float ps = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ps += sacc[tb][i];
      return col_sum4(ps);
    }
  };

  // ---- d = 64 chunk block, both row blocks in one straight-line pass (the
  // products of one row block overlap the softmax of the other): scores
  // relative to the window reference; if any row's sum leaves [2^-100,
  // 2^120] (exp2 overflow or underflow) both are redone against each row's
  // own chunk maximum
  auto chunk_both = [&](const T* sl, const bool (&sel)[2], const float (&sc)[2]) __attribute__((always_inline)) {
    f32x4 sacc[2][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) sacc[cb][tb] = cneg[cb];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FT kf = ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) sacc[cb][tb] = mma16(kf, qf[cb][ks], sacc[cb][tb]);
      }
    }
    FT pf[2][2];
    float ps[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) ps[cb] = chunk_probs(sacc[cb], pf[cb]);
    const bool bad = !(ps[0] >= 0x1p-100f && ps[0] <= 0x1p+120f) || !(ps[1] >= 0x1p-100f && ps[1] <= 0x1p+120f);
    if (__ballot(bad) != 0) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) sacc[cb][tb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const FT kf = ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks);
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) sacc[cb][tb] = mma16(kf, qf[cb][ks], sacc[cb][tb]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        float mx = NEG_INF;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[cb][tb][i]);
        mx = col_max4(mx);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) sacc[cb][tb] -= mx;
        ps[cb] = chunk_probs(sacc[cb], pf[cb]);
      }
    }
    const T* vb = sl + SG::KE;
    f32x4 oc[2][MB];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oc[cb][mb] = zero4();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const FT vf = ld8<T>(vb + (16 * mb + cl) * SG::VP + 8 * gl + 32 * ks);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) oc[cb][mb] = mma16(vf, pf[cb][ks], oc[cb][mb]);
      }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float alpha = sel[cb] ? fast_exp2((sc[cb] - Lr[cb]) * LOG2E) * __builtin_amdgcn_rcpf(ps[cb]) : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] += alpha * oc[cb][mb];
    }
  };

  // ---- chunk block: rows that selected chunk c add exp(s_c - L) O_c
  auto chunk_block = [&](const T* sl, int c) __attribute__((always_inline)) {
    bool sel[2];
    float sc[2];
    unsigned long long anysel = 0;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      sel[cb] = tkc[cbase[cb] + cur[cb]] == c;
      sc[cb] = tks[sbase[cb] + cur[cb]];
      cur[cb] += sel[cb] ? 1 : 0;
    }
    const unsigned long long b0 = __ballot(sel[0]), b1 = __ballot(sel[1]);
    anysel = b0 | b1;
    if (anysel == 0) return;
    if constexpr (FIXREF) {
      chunk_both(sl, sel, sc);
      return;
    }
    FT kf[4][KS];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[tb][ks] = ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks);
    const T* vb = sl + SG::KE;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if ((cb == 0 ? b0 : b1) == 0) continue;
      // d = 64: probabilities relative to the window maximum; a chunk whose
      // scores sit out of fp32 range from it (sum not in [2^-100, 2^120]) is
      // redone with its own maximum, which d = 128 always uses
      f32x4 sacc[4];
      FT pf[2];
      float ps = 0.f;
      bool redo = true;
      if constexpr (FIXREF) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          sacc[tb] = cneg[cb];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sacc[tb] = mma16(kf[tb][ks], qf[cb][ks], sacc[tb]);
        }
        ps = chunk_probs(sacc, pf);
        redo = __ballot(!(ps >= 0x1p-100f && ps <= 0x1p+120f)) != 0;
      }
      if (redo) {
        // (d = 64 reads K from the slot again, so the fragments need not stay
        // live through the common path)
        if constexpr (FIXREF) asm volatile("" ::: "memory");
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          sacc[tb] = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            sacc[tb] = mma16(FIXREF ? ld8<T>(sl + (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks) : kf[tb][ks],
                             qf[cb][ks], sacc[tb]);
        }
        float mx = NEG_INF;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tb][i]);
        mx = col_max4(mx);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) sacc[tb] -= mx;
        ps = chunk_probs(sacc, pf);
      }
      f32x4 oc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oc[mb] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          oc[mb] = mma16(ld8<T>(vb + (16 * mb + cl) * SG::VP + 8 * gl + 32 * ks), pf[ks], oc[mb]);
      const float alpha = sel[cb] ? fast_exp2((sc[cb] - Lr[cb]) * LOG2E) * __builtin_amdgcn_rcpf(ps) : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] += alpha * oc[mb];
    }
  };

  // ------------------------------------------------ pipelined item loop
  if (nW < 2) issue(stg[1], 1);
  commit(stg[0], 0);
  issue(stg[0], 2);
  __syncthreads();
  // one step: publish item n + 1 from register set rg into the other slot
  // (whose item n - 1 every wave has finished), reload rg with item n + 3,
  // then multiply item n. Even items use register set 1, odd items set 0
  // (loops unrolled by two so the sets stay fixed); the window items and the
  // chunk items run in loops of their own.
  auto wstep = [&](int n, u32x4 (&rg)[SG::VPT]) __attribute__((always_inline)) {
    commit(rg, (n + 1) & 1);
    issue(rg, n + 3);
    const T* sl = slots + (n & 1) * SG::ELEMS;
    const int kv0 = kv_lo + 64 * n;
    if (wave_live && kv0 <= pw_hi && kv0 + 63 >= ws_lo) {
      const bool clean = all_valid && kv0 >= ws_hi && kv0 + 63 <= pw_lo;
      if (clean)
        window_block(sl, kv0, std::false_type());
      else
        window_block(sl, kv0, std::true_type());
    }
    __syncthreads();
  };
  auto cstep = [&](int n, u32x4 (&rg)[SG::VPT]) __attribute__((always_inline)) {
    commit(rg, (n + 1) & 1);
    issue(rg, n + 3);
    chunk_block(slots + (n & 1) * SG::ELEMS, __builtin_amdgcn_readfirstlane(ulist[n - nW]));
    __syncthreads();
  };
  int n = 0;
  for (; n + 1 < nW; n += 2) {
    wstep(n, stg[1]);
    wstep(n + 1, stg[0]);
  }
  if (n < nW) wstep(n++, stg[1]);
  fuse();
  auto chunk_loop = [&](u32x4 (&ra)[SG::VPT], u32x4 (&rb)[SG::VPT]) __attribute__((always_inline)) {
    for (; n < NIT; n += 2) {
      cstep(n, ra);
      if (n + 1 >= NIT) break;
      cstep(n + 1, rb);
    }
  };
  if (nW & 1)
    chunk_loop(stg[0], stg[1]);
  else
    chunk_loop(stg[1], stg[0]);

  // ------------------------------------------------ write o and lse
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (prow[cb] < 0) continue;
    const size_t ro = row_off(cb);
    if (gl == 0) lse[ro] = Lr[cb];
    T* dst = o + ro * DH + 4 * gl;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (sizeof(T) == 2) {
        u16x4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = f2bf(oacc[mb][cb][i]);
        *reinterpret_cast<u16x4*>(dst + 16 * mb) = hv;
      } else {
        *reinterpret_cast<f32x4*>(dst + 16 * mb) = oacc[mb][cb];
      }
    }
  }
}

template <typename T, int G, int DH>
static size_t fwd_lds(const Dims& p) {
  constexpr int R = 128, TP = R / G;
  size_t s = sizeof(T) * 2 * (size_t)Slot<T, DH>::ELEMS;
  s += sizeof(int) * (size_t)TP * (p.K + 1) + sizeof(float) * (size_t)R * (p.K + 1);
  s += sizeof(int) * ((size_t)p.C + 1 + std::min<size_t>(p.C, (size_t)TP * p.K));
  return (s + 15) & ~(size_t)15;
}

template <typename T, int G, int DH>
static hipError_t fwd_go(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                         const int32_t* idx, const float* sc, const float* sl, void* o, float* lse,
                         hipStream_t st) {
  constexpr int TP = 128 / G;
  const int ntiles = (p.N + TP - 1) / TP;
  const size_t lds = fwd_lds<T, G, DH>(p);
  auto kern = k_attn_fwd<T, G, DH>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), lds, st, (const T*)q, (const T*)k,
                     (const T*)vt, idx, sc, sl, (T*)o, lse, p.N, Np, p.Hkv, p.K, p.W, p.S, p.scale,
                     ntiles, p.C);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t vt_go(const Dims& p, const void* v, void* vt, int Np, hipStream_t st) {
  hipLaunchKernelGGL((k_vt_perm<T, DH>), dim3(Np / 64, p.B * p.Hkv), dim3(256), 0, st, (const T*)v,
                     (T*)vt, p.N, Np);
  return hipGetLastError();
}

// Strategy: the shared-block kernel streams the union of a tile's selected
// chunks through LDS for all four waves, which pays off when the tile's
// selections concentrate on a modest number of chunks (the tile selects at
// least four times as many slots as there are chunks). Otherwise most
// streamed chunks would serve a single row block, and the bucketed kernel
// (rows of a chunk packed into dense row blocks, chunks taken by waves
// independently) does less work.
// The caller's strategy (Dims::fwd_strategy), or by the rule above when 0:
// 1 shared block; otherwise chunk-major (3, attn_fwd_cm.hip) where its
// envelope allows, else bucketed (2).
int fwd_strategy_of(const Dims& p) {
  if (p.fwd_strategy != 0) return p.fwd_strategy;
  const long tp = 128 / p.G;
  if (tp * p.K >= 4L * p.C) return 1;
  return fwd_cm_ok(p) ? 3 : 2;
}

static bool fwd_use_shared(const Dims& p) { return fwd_strategy_of(p) == 1; }

hipError_t launch_vt_perm(const Dims& p, const void* v, void* vt, hipStream_t st) {
  const int Np = (p.N + 63) / 64 * 64;
  if (p.dtype == 1)
    return p.d == 64 ? vt_go<uint16_t, 64>(p, v, vt, Np, st) : vt_go<uint16_t, 128>(p, v, vt, Np, st);
  return p.d == 64 ? vt_go<float, 64>(p, v, vt, Np, st) : vt_go<float, 128>(p, v, vt, Np, st);
}

template <typename T>
static hipError_t fwd_t(const Dims& p, const void* q, const void* k, const void* vt,
                        const int32_t* idx, const float* sc, const float* sl, void* o, float* lse,
                        hipStream_t st) {
  const int Np = (p.N + 63) / 64 * 64;
  if (fwd_strategy_of(p) == 3) return hipErrorInvalidValue;  // run from the C ABI step by step
  if (!fwd_use_shared(p)) return launch_fwd_sparse(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
  switch (p.G * 1000 + p.d) {
    case 1064: return fwd_go<T, 1, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 1128: return fwd_go<T, 1, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 2064: return fwd_go<T, 2, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 2128: return fwd_go<T, 2, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 4064: return fwd_go<T, 4, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 4128: return fwd_go<T, 4, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static size_t lds_t(const Dims& p) {
  switch (p.G * 1000 + p.d) {
    case 1064: return fwd_lds<T, 1, 64>(p);
    case 1128: return fwd_lds<T, 1, 128>(p);
    case 2064: return fwd_lds<T, 2, 64>(p);
    case 2128: return fwd_lds<T, 2, 128>(p);
    case 4064: return fwd_lds<T, 4, 64>(p);
    case 4128: return fwd_lds<T, 4, 128>(p);
    default: return (size_t)-1;
  }
}

size_t attn_fwd_lds_bytes(const Dims& p) {
  const int strat = fwd_strategy_of(p);
  if (strat == 3) return fwd_cm_ok(p) ? 0 : (size_t)-1;  // checked by fwd_cm_ok
  if (strat == 2) return fwd_sparse_lds_bytes(p);
  const size_t stat = 64;
  return (p.dtype == 1 ? lds_t<uint16_t>(p) : lds_t<float>(p)) + stat;
}

size_t attn_fwd_vt_bytes(const Dims& p) {
  const size_t el = p.dtype == 1 ? 2 : 4;
  return (size_t)p.B * p.Hkv * p.d * ((p.N + 63) / 64 * 64) * el;
}

hipError_t launch_attn_fwd(const Dims& p, const void* q, const void* k, const void* vt,
                           const int32_t* topk_idx, const float* topk_score, const float* sel_lse,
                           void* o, float* lse, hipStream_t st) {
  if (p.dtype == 1) return fwd_t<uint16_t>(p, q, k, vt, topk_idx, topk_score, sel_lse, o, lse, st);
  return fwd_t<float>(p, q, k, vt, topk_idx, topk_score, sel_lse, o, lse, st);
}

}  // namespace hils
