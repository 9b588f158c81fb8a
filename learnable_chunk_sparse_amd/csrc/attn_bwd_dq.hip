// HiLS training backward, dq pass, shared-block strategy (d = 64): the
// counterpart of the forward's shared-block kernel in attn_fwd.hip. Same
// per-row quantities as the bucketed dq pass in attn_bwd.hip (chain rule
// through the fusion with the selection held fixed):
//   window token j:  a_j = exp(x_j - L),  D_W = sum_j a_j (dO . v_j)
//                    U1 = sum_j a_j (dO . v_j) k_j,  U2 = sum_j a_j k_j
//   chunk c:         p_j = softmax of the chunk's scores, delta_c = sum_j p_j (dO . v_j)
//                    w_c = exp(s_c - L),  dx_j = w_c p_j (dO . v_j - delta_c)
//   D = D_W + sum_c w_c delta_c,  dq = scale (U1 - D U2 + sum_c sum_j dx_j k_j)
//   ds_c = w_c (delta_c - D),  dq += scale sum_c ds_c kL_c (the Q-Cal part, dq_hat)
//   beta_c = s_c - L - lse_c and delta_c are kept per (row, slot) for the dk/dv pass.
//
// A tile is 128 rows (128/G positions x G heads) of one (batch, KV head);
// wave w owns rows 32 w .. 32 w + 31 as two 16-row blocks whose U1 (with the
// chunk terms added into it) and U2 accumulators stay in registers, in the
// transposed layout dq^T = K^T dX^T. The tile's work is its window blocks,
// then the union of its rows' selected chunks (ascending); each 64-token
// block's K, V and token-permuted K^T are staged once into one of two LDS
// slots (the next blocks' loads in flight in registers) and read by all four
// waves. Chunk probabilities are taken against the row's L with the shift
// carried in the MFMA accumulator; a row block whose sum leaves [2^-100,
// 2^120] is redone against the chunk's own maximum.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

template <typename T, int DH>
struct BSlot {
  static constexpr int VE = 16 / (int)sizeof(T);
  static constexpr int KP = DH + VE;        // K and V row pitch
  static constexpr int TP2 = 64 + VE;       // K^T row pitch
  static constexpr int KE = 64 * KP;        // K (then V) part
  static constexpr int ELEMS = 2 * KE + DH * TP2;
  static constexpr int NV = 64 * DH / VE;   // 16-byte vectors of each of K, V, K^T
  static constexpr int VPT = 3 * NV / 256;  // per thread
};

template <typename T, int G, int DH>
__global__ __launch_bounds__(256, 2) void k_bwd_dq_sh(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ kt, int Np, const T* __restrict__ dO, const T* __restrict__ kL,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ sT,
    const float* __restrict__ lse, float* __restrict__ Dv, float* __restrict__ dq,
    float* __restrict__ dqhat, float* __restrict__ ds_o, float* __restrict__ beta_o,
    float* __restrict__ delta_o, int N, int Hkv, int K, int W, int S, float scale, int ntiles,
    int C) {
  typedef typename Frag<T>::type FT;
  typedef BSlot<T, DH> SG;
  constexpr int R = 128, TP = R / G;
  constexpr int KS = DH / 32, MB = DH / 16;
  constexpr int RS = DH + 4;  // accumulator row pitch in the epilogue

  extern __shared__ __align__(16) unsigned char smem[];
  T* slots = reinterpret_cast<T*>(smem);                    // [2][ELEMS]
  const int K1 = K + 1;                                     // lists end with a sentinel
  int* tkc = reinterpret_cast<int*>(slots + 2 * SG::ELEMS); // [TP][K + 1] selected chunks
  float* lw = reinterpret_cast<float*>(tkc + TP * K1);      // [R][K + 1] s_c - L (-inf: none)
  int* flg = reinterpret_cast<int*>(lw + R * K1);           // [C + 1]
  int* ulist = flg + C + 1;                                 // union, ascending
  // epilogue (the slots are free by then): dq^T part per row, D per row, ds
  float* accS = reinterpret_cast<float*>(smem);             // [R][RS]
  float* Ds = accS + R * RS;                                // [R]
  float* dsS = Ds + R;                                      // [R][K]
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
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)bg * N * DH, N * DH * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (size_t)bg * N * DH, N * DH * (int)sizeof(T));
  const __amdgpu_buffer_rsrc_t trs = make_rsrc(kt + (size_t)bg * DH * Np, DH * Np * (int)sizeof(T));
  const float sc2 = scale * LOG2E;

  // ------------------------------------------------ per-lane rows
  FT qf[2][KS], df[2][KS];
  int prow[2], wsr[2], cbase[2], sbase[2], cur[2];
  float Lr[2];
  auto row_off = [&](int cb) __attribute__((always_inline)) -> size_t {
    const int r = 32 * w + 16 * cb + cl;
    const int pos = min(p0 + r / G, N - 1);
    return ((size_t)b * Hq + g * G + r % G) * N + pos;
  };
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int r = 32 * w + 16 * cb + cl;
    const int pos = p0 + r / G;
    cbase[cb] = (r / G) * K1;
    sbase[cb] = r * K1;
    prow[cb] = pos < N ? pos : -1;
    wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
    cur[cb] = 0;
    const size_t ro = row_off(cb);
    Lr[cb] = lse[ro];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[cb][ks] = ld8<T>(q + ro * DH + 8 * gl + 32 * ks);
      df[cb][ks] = ld8<T>(dO + ro * DH + 8 * gl + 32 * ks);
    }
  }
  const int pw_lo = p0 + 32 * w / G;
  const int pw_hi = min(p0 + (32 * w + 31) / G, N - 1);
  const bool wave_live = pw_lo < N;
  const bool all_valid = p0 + (32 * w + 31) / G < N;
  const int ws_lo = wave_live ? n_distant(pw_lo, W, S) * S : 0;
  const int ws_hi = wave_live ? n_distant(pw_hi, W, S) * S : 0;

  // acc1: U1 plus the chunk terms, acc2: U2 (rows d = 16 mb + 4 gl + i, column = row)
  f32x4 acc1[MB][2], acc2[MB][2];
  float dw[2], dc[2];
  f32x4 cneg[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    dw[cb] = 0.f;
    dc[cb] = 0.f;
    const float lr = prow[cb] >= 0 ? -Lr[cb] / scale : 0.f;  // -L in raw score units
    cneg[cb] = f32x4{lr, lr, lr, lr};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc1[mb][cb] = zero4();
      acc2[mb][cb] = zero4();
    }
  }

  // ------------------------------------------------ block staging
  const int kv_lo = n_distant(p0, W, S) * S;
  const int nW = (plast - kv_lo) / 64 + 1;
  u32x4 stg[SG::VPT];  // the next block's vectors, in flight during the current block
  auto issue_kv = [&](u32x4 (&rg)[SG::VPT], int kv0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < SG::VPT; ++s) {
      const int vi = tid + 256 * s;
      const int part = vi / SG::NV, vj = vi - part * SG::NV;
      if (part < 2) {
        const int tok = vj / (DH / SG::VE), pp = vj - tok * (DH / SG::VE);
        rg[s] = buf_ld16(part == 0 ? krs : vrs, ((kv0 + tok) * DH + pp * SG::VE) * (int)sizeof(T));
      } else {
        const int dd = vj / (64 / SG::VE), pp = vj - dd * (64 / SG::VE);
        rg[s] = buf_ld16(trs, (dd * Np + kv0 + pp * SG::VE) * (int)sizeof(T));
      }
    }
  };
  auto commit = [&](const u32x4 (&rg)[SG::VPT], int slot) __attribute__((always_inline)) {
    T* base = slots + slot * SG::ELEMS;
#pragma unroll
    for (int s = 0; s < SG::VPT; ++s) {
      const int vi = tid + 256 * s;
      const int part = vi / SG::NV, vj = vi - part * SG::NV;
      T* dst;
      if (part < 2) {
        const int tok = vj / (DH / SG::VE), pp = vj - tok * (DH / SG::VE);
        dst = base + part * SG::KE + tok * SG::KP + pp * SG::VE;
      } else {
        const int dd = vj / (64 / SG::VE), pp = vj - dd * (64 / SG::VE);
        dst = base + 2 * SG::KE + dd * SG::TP2 + pp * SG::VE;
      }
      *reinterpret_cast<u32x4*>(dst) = rg[s];
    }
  };
  issue_kv(stg, kv_lo);

  // ------------------------------------------------ selections of the tile
  for (int x = tid; x <= ndmax; x += 256) flg[x] = 0;
  {
    // ids [TP][K] and scores [R][K]: 16-byte vectors requested before use
    const int KV4 = K >> 2, nvi = TP * KV4, nvs = R * KV4;
    int4 vi[4];
    f32x4 vs[4];
    float lv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vv = tid + 256 * j;
      const int vc = min(vv, nvi - 1), rc = vc / KV4, pc = vc - rc * KV4;
      vi[j] = *reinterpret_cast<const int4*>(topk_idx + ((size_t)bg * N + min(p0 + rc, N - 1)) * K + 4 * pc);
      const int ws2 = min(vv, nvs - 1), rs = ws2 / KV4, qs2 = ws2 - rs * KV4;
      const size_t ro = ((size_t)b * Hq + g * G + rs % G) * N + min(p0 + rs / G, N - 1);
      vs[j] = *reinterpret_cast<const f32x4*>(sT + ro * K + 4 * qs2);
      lv[j] = lse[ro];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vv = tid + 256 * j;
      if (vv < nvi) {
        const int r = vv / KV4, part = vv - r * KV4;
        const bool li = p0 + r < N;
        int* dcp = tkc + r * K1 + 4 * part;
        dcp[0] = li ? vi[j].x : -1;
        dcp[1] = li ? vi[j].y : -1;
        dcp[2] = li ? vi[j].z : -1;
        dcp[3] = li ? vi[j].w : -1;
      }
    }
    for (int x = tid; x < TP; x += 256) tkc[x * K1 + K] = -1;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int vv = tid + 256 * j;
      if (vv < nvs) {
        const int r = vv / KV4, part = vv - r * KV4;
        const int* tc = tkc + (r / G) * K1 + 4 * part;
        float* dl = lw + r * K1 + 4 * part;
#pragma unroll
        for (int i = 0; i < 4; ++i) dl[i] = tc[i] >= 0 ? vs[j][i] - lv[j] : NEG_INF;
      }
    }
    for (int x = tid; x < R; x += 256) lw[x * K1 + K] = NEG_INF;
  }
  __syncthreads();
  for (int x = tid; x < TP * K1; x += 256) {
    const int c = tkc[x];
    if (c >= 0 && c < ndmax) flg[c] = 1;
  }
  __syncthreads();
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

  // S^T = K Q^T and dP^T = V dO^T of one row block (rows = tokens)
  auto scores = [&](const T* sl, int cb, f32x4 (&sa)[4], f32x4 (&pa)[4], const f32x4& c0) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      sa[tb] = c0;
      pa[tb] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int o = (16 * tb + cl) * SG::KP + 8 * gl + 32 * ks;
        sa[tb] = mma16(ld8<T>(sl + o), qf[cb][ks], sa[tb]);
        pa[tb] = mma16(ld8<T>(sl + SG::KE + o), df[cb][ks], pa[tb]);
      }
    }
  };
  // acc += K^T X^T for a token block X^T in D layout (rows = tokens)
  auto ktprod = [&](const T* sl, const f32x4 (&x)[4], f32x4 (&acc)[MB][2], int cb) __attribute__((always_inline)) {
    const T* tb2 = sl + 2 * SG::KE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const FT xf = pk8<T>(x[2 * ks], x[2 * ks + 1]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb][cb] = mma16(ld8<T>(tb2 + (16 * mb + cl) * SG::TP2 + 8 * gl + 32 * ks), xf, acc[mb][cb]);
    }
  };

  // ---- window block: a_j = exp(x_j - L) (masked), U1, U2, D_W
  auto window_block = [&](const T* sl, int kv0, auto masked) __attribute__((always_inline)) {
    constexpr bool MSK = decltype(masked)::value;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      // fragments are re-read from LDS per row block (registers, not LDS
      // bandwidth, are the scarce resource here)
      asm volatile("" ::: "memory");
      f32x4 sa[4], pa[4];
      scores(sl, cb, sa, pa, zero4());
      const float lb = Lr[cb] * LOG2E;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = fast_exp2(fmaf(sa[tb][i], sc2, -lb));
          if constexpr (MSK) {
            const int j = kv0 + 16 * tb + 4 * gl + i;
            a = (j <= prow[cb] && j >= wsr[cb]) ? a : 0.f;
          }
          const float adp = a * pa[tb][i];
          dw[cb] += adp;
          sa[tb][i] = a;
          pa[tb][i] = adp;
        }
      ktprod(sl, pa, acc1, cb);
      ktprod(sl, sa, acc2, cb);
    }
  };

  // ---- chunk block: rows that selected chunk c
  auto chunk_block = [&](const T* sl, int c) __attribute__((always_inline)) {
    bool sel[2];
    float lwv[2];
    int slot[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      sel[cb] = tkc[cbase[cb] + cur[cb]] == c;
      lwv[cb] = lw[sbase[cb] + cur[cb]];
      slot[cb] = cur[cb];
      cur[cb] += sel[cb] ? 1 : 0;
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (__ballot(sel[cb]) == 0) continue;
      asm volatile("" ::: "memory");
      f32x4 sa[4], pa[4];
      scores(sl, cb, sa, pa, cneg[cb]);
      // probabilities against L (e_j = exp(x_j - L)); ref = the shift in nats
      float ps = 0.f, ed = 0.f, ref = Lr[cb];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(sa[tb][i] * sc2);
          sa[tb][i] = e;
          ps += e;
          ed = fmaf(e, pa[tb][i], ed);
        }
      ps = col_sum4(ps);
      if (__ballot(!(ps >= 0x1p-100f && ps <= 0x1p+120f)) != 0) {
        // out of range against L: the chunk's own maximum instead
        asm volatile("" ::: "memory");
        scores(sl, cb, sa, pa, zero4());
        float mx = NEG_INF;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sa[tb][i]);
        mx = col_max4(mx);
        ref = mx * scale;
        ps = 0.f;
        ed = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2((sa[tb][i] - mx) * sc2);
            sa[tb][i] = e;
            ps += e;
            ed = fmaf(e, pa[tb][i], ed);
          }
        ps = col_sum4(ps);
      }
      ed = col_sum4(ed);
      const float rps = __builtin_amdgcn_rcpf(ps);
      const float dlt = ed * rps;
      const float wc = sel[cb] ? fast_exp2(lwv[cb] * LOG2E) : 0.f;
      const float f = wc * rps;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[tb][i] = f * sa[tb][i] * (pa[tb][i] - dlt);
      ktprod(sl, sa, acc1, cb);
      if (sel[cb]) {
        dc[cb] = fmaf(wc, dlt, dc[cb]);
        if (gl == 0) {
          const size_t o = row_off(cb) * K + slot[cb];
          beta_o[o] = lwv[cb] - (ref + __logf(ps));
          delta_o[o] = dlt;
        }
      }
    }
  };

  // ------------------------------------------------ item loops
  // step n: publish block n + 1 (in registers) into the slot block n - 1
  // used, request block n + 2, multiply block n
  commit(stg, 0);
  issue(stg, 1);
  __syncthreads();
  for (int n = 0; n < nW; ++n) {
    commit(stg, (n + 1) & 1);
    issue(stg, n + 2);
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
  }
  for (int n = nW; n < NIT; ++n) {
    commit(stg, (n + 1) & 1);
    issue(stg, n + 2);
    chunk_block(slots + (n & 1) * SG::ELEMS, __builtin_amdgcn_readfirstlane(ulist[n - nW]));
    __syncthreads();
  }

  // ------------------------------------------------ D, dq token part, ds
  // (every wave has passed the last barrier: the slots are free)
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float D = col_sum4(dw[cb]) + dc[cb];
    const int r = 32 * w + 16 * cb + cl;
    if (gl == 0) {
      Ds[r] = D;
      if (prow[cb] >= 0) Dv[row_off(cb)] = D;
    }
    float* dst = accS + r * RS + 4 * gl;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      *reinterpret_cast<f32x4*>(dst + 16 * mb) = scale * (acc1[mb][cb] - D * acc2[mb][cb]);
  }
  __syncthreads();
  {
    constexpr int XB = 8;
    for (int x0 = 0; x0 < R * K; x0 += 256 * XB) {
      float dl[XB];
#pragma unroll
      for (int j = 0; j < XB; ++j) {
        const int x = min(x0 + tid + 256 * j, R * K - 1);
        const int r = x / K, kk = x - r * K;
        const int pos = min(p0 + r / G, N - 1);
        dl[j] = delta_o[(((size_t)b * Hq + g * G + r % G) * N + pos) * K + kk];
      }
#pragma unroll
      for (int j = 0; j < XB; ++j) {
        const int x = x0 + tid + 256 * j;
        if (x >= R * K) continue;
        const int r = x / K, kk = x - r * K;
        const int pos = p0 + r / G;
        const float lwx = lw[r * K1 + kk];
        const float dsv = (pos < N && lwx != NEG_INF) ? fast_exp2(lwx * LOG2E) * (dl[j] - Ds[r]) : 0.f;
        dsS[x] = dsv;
        if (pos < N) ds_o[(((size_t)b * Hq + g * G + r % G) * N + pos) * K + kk] = dsv;
      }
    }
  }
  __syncthreads();
  // dq = token part + scale sum_c ds_c kL_c (chunk ids and landmark rows in
  // batches of eight, requested at once)
  for (int x = tid; x < R * DH / 4; x += 256) {
    const int r = x / (DH / 4), d4 = 4 * (x - r * (DH / 4));
    const int pos = p0 + r / G, hh = r % G;
    if (pos >= N) continue;
    const int* ti = tkc + (r / G) * K1;
    f32x4 sur = zero4();
    for (int k0 = 0; k0 < K; k0 += 8) {
      int cc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) cc[j] = ti[min(k0 + j, K - 1)];
      float kv[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const T* kr = kL + ((size_t)bg * C + (cc[j] >= 0 ? cc[j] : 0)) * DH + d4;
        if constexpr (sizeof(T) == 2) {
          const u16x4 hv = *reinterpret_cast<const u16x4*>(kr);
#pragma unroll
          for (int i = 0; i < 4; ++i) kv[j][i] = bf2f(hv[i]);
        } else {
          const f32x4 fv = *reinterpret_cast<const f32x4*>(kr);
#pragma unroll
          for (int i = 0; i < 4; ++i) kv[j][i] = fv[i];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool ok = k0 + j < K && cc[j] >= 0;
        const float dsv = ok ? dsS[r * K + min(k0 + j, K - 1)] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) sur[i] += dsv * kv[j][i];
      }
    }
    sur *= scale;
    const f32x4 tok = *reinterpret_cast<const f32x4*>(accS + r * RS + d4);
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pos;
    *reinterpret_cast<f32x4*>(dq + ro * DH + d4) = tok + sur;
    if (dqhat != nullptr) *reinterpret_cast<f32x4*>(dqhat + ro * DH + d4) = sur;
  }
}

template <typename T, int G, int DH>
static size_t dqsh_lds_g(const Dims& p) {
  constexpr int R = 128, TP = R / G;
  size_t s = sizeof(T) * 2 * (size_t)BSlot<T, DH>::ELEMS;
  s += sizeof(int) * (size_t)TP * (p.K + 1) + sizeof(float) * (size_t)R * (p.K + 1);
  s += sizeof(int) * ((size_t)p.C + 1 + std::min<size_t>(p.C, (size_t)TP * p.K));
  const size_t epi = sizeof(float) * ((size_t)R * (DH + 4) + R + (size_t)R * p.K);
  return (std::max(s, epi) + 15) & ~(size_t)15;
}

static size_t dqsh_lds(const Dims& p) {
  switch (p.G) {
    case 1: return dqsh_lds_g<uint16_t, 1, 64>(p);
    case 2: return dqsh_lds_g<uint16_t, 2, 64>(p);
    case 4: return dqsh_lds_g<uint16_t, 4, 64>(p);
    default: return (size_t)-1;
  }
}

// The shared-block dq pass serves bf16, d = 64, K a multiple of 4 (at most
// 32), tiles whose selections concentrate (the tile selects at least four
// times as many slots as there are chunks, as for the forward's choice) and
// two tiles per CU of LDS.
bool bwd_dq_shared_ok(const Dims& p) {
  if (p.dtype != 1 || p.d != 64 || p.K % 4 != 0 || p.K > 32) return false;
  if ((128L / p.G) * p.K < 4L * p.C) return false;
  return dqsh_lds(p) <= 80 * 1024;
}

template <int G>
static hipError_t dqsh_go(const Dims& p, const void* q, const void* k, const void* v, const void* kt,
                          int Np, const void* dO, const void* kL, const int32_t* topk_idx,
                          const float* sT, const float* lse, float* Dv, float* dq, float* dqhat,
                          float* ds, float* beta, float* delta, hipStream_t st) {
  constexpr int TP = 128 / G;
  const int ntiles = (p.N + TP - 1) / TP;
  const size_t lds = dqsh_lds(p);
  auto kern = k_bwd_dq_sh<uint16_t, G, 64>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), lds, st, (const uint16_t*)q,
                     (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)kt, Np,
                     (const uint16_t*)dO, (const uint16_t*)kL, topk_idx, sT, lse, Dv, dq, dqhat, ds,
                     beta, delta, p.N, p.Hkv, p.K, p.W, p.S, p.scale, ntiles, p.C);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_shared(const Dims& p, const void* q, const void* k, const void* v,
                                const void* kt, int Np, const void* dO, const void* kL,
                                const int32_t* topk_idx, const float* sT, const float* lse,
                                float* Dv, float* dq, float* dqhat, float* ds, float* beta,
                                float* delta, hipStream_t st) {
  switch (p.G) {
    case 1: return dqsh_go<1>(p, q, k, v, kt, Np, dO, kL, topk_idx, sT, lse, Dv, dq, dqhat, ds, beta, delta, st);
    case 2: return dqsh_go<2>(p, q, k, v, kt, Np, dO, kL, topk_idx, sT, lse, Dv, dq, dqhat, ds, beta, delta, st);
    case 4: return dqsh_go<4>(p, q, k, v, kt, Np, dO, kL, topk_idx, sT, lse, Dv, dq, dqhat, ds, beta, delta, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hils
