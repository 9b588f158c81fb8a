// HiLS training backward (paper Fig. 3 caption: the chunk-mass surrogate
// parameterises the forward attention weights, so the language-modelling
// gradient reaches the compressed keys; dev.to / nestfrontier: gradients flow
// into the landmark representations through the fusion). The pages print no
// backward formulas; these are the chain rule through the forward with the
// selection T held fixed. Per row (b, h, i), with O the forward output,
// L its log-normaliser, w_c = exp(s_c - L), p_j = softmax within chunk c:
//   D = dO . O,  delta_c = dO . O_c = sum_j p_j (dO . v_j)
//   chunk token j:  a_j = w_c p_j,         dx_j = a_j (dO . v_j - delta_c)
//   window token j: a_j = exp(x_j - L),    dx_j = a_j (dO . v_j - D)
//   dq += scale sum_j dx_j k_j;  dk_j += scale dx_j q;  dv_j += a_j dO
//   ds_c = w_c (delta_c - D):  dq_hat = scale sum_c ds_c kL_c (added to dq),
//   dkL_c += scale ds_c q_hat,  de_c += ds_c
//   Q-Cal: d(delta q) = dq_hat, du = W_up^T dq_hat, dW_up += dq_hat u^T,
//   dW_down += du h^T, dh += W_down^T du.
//
// Launch sequence:
//   (Q-Cal forward again for q_hat and u)
//   k_bwd_prep     D per row and the fp32 scores s_c of the selected chunks
//   inverse index  chunk -> (position, slot) lists (count, scan, fill)
//   k_bwd_dq       query tiles: window band + compacted chunk groups (as in
//                  the forward), dq; per (row, chunk) ds_c, beta_c = s_c - L -
//                  lse_c (so that a_j = exp(x_j + beta_c)) and delta_c
//   k_bwd_dkdv     one workgroup per 64-token key block: every row attending
//                  to it through the window or through a selection; dk, dv
//                  and (complete chunks) dkL, de, without atomics to HBM
//   Q-Cal backward on the batched MFMA GEMM.
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

// token-permuted transposed copy of a [N][d] tensor (defined with the forward)
template <typename T, int DH>
__global__ void k_vt_perm(const T* __restrict__ v, T* __restrict__ vt, int N, int Np);

// --------------------------------------------------------------- small kernels
__global__ void k_fill_f32(float* __restrict__ p, size_t n, float v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// fp32 score s_c = scale q_hat . kL_c + e_c of every selected slot. A
// workgroup takes 64 consecutive query rows: their q_hat rows and their
// (row, slot) chunk ids are staged in LDS together (one round trip), then
// eight adjacent lanes share a (row, slot) pair, each reading DH / 8 elements
// of the selected landmark row (one wave load covers eight whole rows, which
// stay in L2), with all of a lane's landmark loads in flight at once; the
// partial dot products are summed across the eight lanes.
template <typename T, typename QT, int DH>
__global__ __launch_bounds__(256) void k_bwd_prep(const QT* __restrict__ qs, const T* __restrict__ kL,
                                                  const T* __restrict__ e,
                                                  const int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ sT, long rows, int N, int Hq,
                                                  int Hkv, int G, int C, int K, float scale) {
  constexpr int PR = 64, QP = DH + 4, DL = DH / 8, NF = DL / 8, UP = 8, KMAX = 32;
  typedef typename Frag<T>::type FT;
  __shared__ __align__(16) float qrow[PR * QP];
  __shared__ int cid[PR * KMAX];  // chunk id of pair x = row * K + slot
  __shared__ long cbase[PR];      // bg C: the row's landmark rows
  const int tid = threadIdx.x;
  const long r0 = (long)blockIdx.x * PR;
  const int nrow = (int)std::min<long>(PR, rows - r0);
  const int npair = nrow * K;
  // x / K for pair ids x < 2^11 through a float reciprocal: (x + 1/2) / K
  // lies at least 1/(2K) away from an integer, far beyond the rounding
  const float invK = 1.f / (float)K;
  auto row_idx = [&](int x) __attribute__((always_inline)) { return (int)(((float)x + 0.5f) * invK); };
  // (b, h, i) of the first row; rows r0 + rr follow it
  const long bh0 = r0 / N;
  const int i0 = (int)(r0 - bh0 * N), h0 = (int)(bh0 % Hq), b0 = (int)(bh0 / Hq);
  auto row_of = [&](int rr, long& bg, int& i) __attribute__((always_inline)) {
    int ii = i0 + rr, h = h0, b = b0;
    while (ii >= N) {
      ii -= N;
      if (++h == Hq) h = 0, ++b;
    }
    bg = (long)b * Hkv + h / G;
    i = ii;
  };
  for (int x = tid; x < npair; x += 256) {
    const int rr = row_idx(x), kk = x - rr * K;
    long bg;
    int i;
    row_of(rr, bg, i);
    cid[x] = topk_idx[(bg * N + i) * K + kk];
  }
  if (tid < nrow) {
    long bg;
    int i;
    row_of(tid, bg, i);
    cbase[tid] = bg * C;
  }
  for (int x = tid; x < PR * DH / 4; x += 256) {
    const int rr = x / (DH / 4), d4 = 4 * (x - rr * (DH / 4));
    const long row = r0 + rr;
    f32x4 v = zero4();
    if (row < rows) {
      if constexpr (sizeof(QT) == 4) {
        v = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(qs) + row * DH + d4);
      } else {
        const u16x4 h4 = *reinterpret_cast<const u16x4*>(qs + row * DH + d4);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = bf2f(h4[j]);
      }
    }
    *reinterpret_cast<f32x4*>(qrow + rr * QP + d4) = v;
  }
  __syncthreads();
  const int l8 = tid & 7, pr = tid >> 3;  // 32 pairs per pass
  for (int x0 = pr; x0 < npair; x0 += 32 * UP) {
    FT kv[UP][NF];
    float ev[UP];
    int cc[UP];
#pragma unroll
    for (int t = 0; t < UP; ++t) {
      const int x = min(x0 + 32 * t, npair - 1);
      cc[t] = cid[x];
      const long kc = cbase[row_idx(x)] + max(cc[t], 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) kv[t][f] = ld8<T>(kL + kc * DH + DL * l8 + 8 * f);
      ev[t] = to_f<T>(e[kc]);
    }
#pragma unroll
    for (int t = 0; t < UP; ++t) {
      const int x = x0 + 32 * t;
      const float* qr = qrow + row_idx(min(x, npair - 1)) * QP + DL * l8;
      float acc = 0.f;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const f32x4 qa = *reinterpret_cast<const f32x4*>(qr + 8 * f);
        const f32x4 qb = *reinterpret_cast<const f32x4*>(qr + 8 * f + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc = fmaf(qa[j], (float)kv[t][f][j], acc);
          acc = fmaf(qb[j], (float)kv[t][f][j + 4], acc);
        }
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      if (l8 == 0 && x < npair)
        sT[r0 * K + x] = cc[t] >= 0 ? fmaf(acc, scale, ev[t]) : __builtin_nanf("");
    }
  }
}

// --------------------------------------------------------------- helpers

__device__ int bwd_block_scan(int* a, int n, int* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int seg = (n + 255) / 256;
  const int lo = min(n, t * seg), hi = min(n, lo + seg);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += a[i];
  int v = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  int base = v - s;
  for (int j = 0; j < w; ++j) base += wsum[j];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  for (int i = lo; i < hi; ++i) {
    const int x = a[i];
    a[i] = base;
    base += x;
  }
  __syncthreads();
  return total;
}

// --------------------------------------------------------------- dq pass
// D = dO . O is not taken from the rounded output o: with a_j the forward
// weights, D = sum_window a_j (dO . v_j) + sum_c w_c delta_c exactly, so the
// chunks are processed first (their terms do not involve D), then the window
// accumulates U1 = sum a_j (dO . v_j) k_j and U2 = sum a_j k_j so that its dq
// part scale (U1 - D U2) is formed once D is known.
// As in the forward, S^T = K Q^T and dP^T = V dO^T keep the probabilities in
// the operand layout of dq^T = K^T dS^T, with K^T read from a token-permuted
// transposed copy; waves take whole chunks dynamically and add into private
// accumulator copies (no LDS atomics on the d-vectors).
template <typename T, int DH>
struct BwdChunkFrags {
  typename Frag<T>::type k[4][DH / 32];   // K rows (A of S^T)
  typename Frag<T>::type v[4][DH / 32];   // V rows (A of dP^T)
  typename Frag<T>::type kt[DH / 16][2];  // K^T rows (A of dq^T)
};

template <typename T, int DH>
__device__ __forceinline__ void bwd_load_block(BwdChunkFrags<T, DH>& f, const T* __restrict__ kb,
                                               const T* __restrict__ vb, int nvalid,
                                               const T* __restrict__ ktb, int Np, int lane) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    int tok = 16 * tb + (lane & 15);
    tok = tok < nvalid ? tok : 0;
    const size_t o = (size_t)tok * DH + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
      f.k[tb][ks] = ld8<T>(kb + o + 32 * ks);
      f.v[tb][ks] = ld8<T>(vb + o + 32 * ks);
    }
  }
#pragma unroll
  for (int mb = 0; mb < DH / 16; ++mb) {
    const T* src = ktb + (size_t)(16 * mb + (lane & 15)) * Np + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) f.kt[mb][ks] = ld8<T>(src + 32 * ks);
  }
}

template <typename T, int G, int DH, int CB>
__global__ __launch_bounds__(256) void k_bwd_dq(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ kt, int Np, const T* __restrict__ dO, const T* __restrict__ kL,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ sT,
    const float* __restrict__ lse, float* __restrict__ Dv, float* __restrict__ dq,
    float* __restrict__ dqhat, float* __restrict__ ds_o, float* __restrict__ beta_o,
    float* __restrict__ delta_o, int N, int Hkv, int K, int W, int S, float scale, int ntiles,
    int C) {
  typedef typename Frag<T>::type FT;
  constexpr int R = 64 * CB, TP = R / G;
  constexpr int KS = DH / 32, MB = DH / 16;
  constexpr int RS = DH + 4;  // accumulator row stride
  constexpr int EPT = TP * 32 / 256;
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = TP * K;                             // the tile's (position, slot) entries
  int NE = 1;                                       // E rounded up to a power of two
  while (NE < E) NE <<= 1;
  float* accT = reinterpret_cast<float*>(smem);     // [4][R][RS] per-wave copies
  float* Ls = accT + 4 * R * RS;                    // [R]
  float* Ds = Ls + R;                               // [R] chunk part of D, then D
  float* dsS = Ds + R;                              // [R][K] fusion weights
  float* dlS = dsS + R * K;                         // [R][K] delta_c of each slot
  // the tile's selections sorted by (chunk, entry), then grouped into runs
  uint32_t* skey = reinterpret_cast<uint32_t*>(dlS + R * K);  // [NE] sorted keys
  int* rfl = reinterpret_cast<int*>(skey + NE);               // [NE] run heads -> run index
  int* rch = rfl + NE;                                        // [NE] chunk of each run
  int* rst = rch + NE;                                        // [NE + 1] first entry of each run
  uint16_t* ent = reinterpret_cast<uint16_t*>(rst + NE + 1);  // [NE] entries in key order
  __shared__ int wsum[4];
  __shared__ int etot;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int tx, bg;
  xcd_block(tx, bg);
  const int tile = ntiles - 1 - tx;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * TP;
  const int plast = min(p0 + TP - 1, N - 1);
  const int ndmax = n_distant(plast, W, S);
  const T* kg = k + (size_t)bg * N * DH;
  const T* vg = v + (size_t)bg * N * DH;
  const T* ktg = kt + (size_t)bg * DH * Np;
  float* accW = accT + w * R * RS;

  for (int x = tid; x < R * RS; x += 256) reinterpret_cast<f32x4*>(accT)[x] = zero4();
  for (int x = tid; x < R; x += 256) {
    const int pos = p0 + x / G, hh = x % G;
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + (pos < N ? pos : N - 1);
    Ls[x] = lse[ro];
    Ds[x] = 0.f;
  }
  for (int x = tid; x < R * K; x += 256) {
    dsS[x] = 0.f;
    dlS[x] = 0.f;
  }
  // group the tile's selections by chunk: keys (chunk << 12 | entry), absent
  // ones last, sorted by a bitonic network in LDS (no per-chunk table, so no
  // bound on the number of chunks; the order is a function of the data)
  if (tid == 0) etot = 0;
  int my_c[EPT];
  // all of the thread's ids are requested before any is used (clamped
  // addresses; guarded per-element loads would each wait for the previous)
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int x = min(tid + 256 * j, E - 1);
    const int pl = x / K, kk = x - pl * K;
    my_c[j] = topk_idx[((size_t)bg * N + min(p0 + pl, N - 1)) * K + kk];
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int x = tid + 256 * j;
    const int c = my_c[j];
    const bool ok = x < E && p0 + x / K < N && c >= 0 && c < ndmax;
    if (x < NE) skey[x] = ok ? ((uint32_t)c << 12) | (uint32_t)x : 0xFFFFFFFFu;
  }
  for (int x = EPT * 256 + tid; x < NE; x += 256) skey[x] = 0xFFFFFFFFu;
  __syncthreads();
  for (int kb = 2; kb <= NE; kb <<= 1)
    for (int jb = kb >> 1; jb > 0; jb >>= 1) {
      for (int i = tid; i < NE; i += 256) {
        const int l = i ^ jb;
        if (l > i) {
          const uint32_t a = skey[i], bb = skey[l];
          if ((a > bb) == ((i & kb) == 0)) {
            skey[i] = bb;
            skey[l] = a;
          }
        }
      }
      __syncthreads();
    }
  // runs of one chunk: heads flagged, exclusive scan gives each head its run
  int nvalid = 0;
  for (int i = tid; i < NE; i += 256) {
    const uint32_t key = skey[i];
    const bool ok = key != 0xFFFFFFFFu;
    const int x = (int)(key & 0xFFFu), pl = x / K, kk = x - pl * K;
    ent[i] = (uint16_t)((pl << 6) | kk);
    rfl[i] = ok && (i == 0 || (skey[i - 1] >> 12) != (key >> 12)) ? 1 : 0;
    nvalid += ok ? 1 : 0;
  }
  atomicAdd(&etot, nvalid);  // integer sum: order-free
  __syncthreads();
  const int NZ = bwd_block_scan(rfl, NE, wsum);
  // run r: chunk rch[r], entries rst[r] .. rst[r + 1] - 1 of ent
  for (int i = tid; i < NE; i += 256) {
    const uint32_t key = skey[i];
    if (key != 0xFFFFFFFFu && (i == 0 || (skey[i - 1] >> 12) != (key >> 12))) {
      rch[rfl[i]] = (int)(key >> 12);
      rst[rfl[i]] = i;
    }
  }
  if (tid == 0) rst[NZ] = etot;
  __syncthreads();

  const float sc2 = scale * LOG2E;
  // ---------------- selected chunks (terms free of D)
  {
    // runs taken round-robin (a fixed assignment: each row's chunk terms are
    // summed in the same order on every run)
    BwdChunkFrags<T, DH> f;
    for (int a = w; a < NZ; a += 4) {
      const int c = rch[a];
      const int e0 = rst[a], n = rst[a + 1] - e0;
      bwd_load_block<T, DH>(f, kg + (size_t)c * 64 * DH, vg + (size_t)c * 64 * DH, 64, ktg + (size_t)c * 64, Np, lane);
      const int nb = (n * G + 15) / 16;
      for (int cbk = 0; cbk < nb; ++cbk) {
        const int rr = 16 * cbk + (lane & 15);
        const bool valid = rr < n * G;
        const int ei = (valid ? rr : 0) / G, hh = (valid ? rr : 0) % G;
        const int en = ent[e0 + ei];
        const int pl = en >> 6, kk = en & 63;
        const int row = pl * G + hh;
        const size_t ro = ((size_t)b * Hq + g * G + hh) * N + p0 + pl;
        FT qf[KS], df[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qf[ks] = ld8<T>(q + ro * DH + 8 * (lane >> 4) + 32 * ks);
          df[ks] = ld8<T>(dO + ro * DH + 8 * (lane >> 4) + 32 * ks);
        }
        const float sc = valid ? sT[ro * K + kk] : 0.f;
        f32x4 sa[4], pa[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          sa[tb] = zero4();
          pa[tb] = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            sa[tb] = mma16(f.k[tb][ks], qf[ks], sa[tb]);
            pa[tb] = mma16(f.v[tb][ks], df[ks], pa[tb]);
          }
        }
        float mx = NEG_INF;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sa[tb][i]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mref = mx * sc2;
        float ls = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = fast_exp2(fmaf(sa[tb][i], sc2, -mref));
            sa[tb][i] = pv;
            ls += pv;
          }
        ls += shfl_xor(ls, 16);
        ls += shfl_xor(ls, 32);
        const float inv = 1.f / ls;
        float dl = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sa[tb][i] *= inv;  // p within the chunk
            dl += sa[tb][i] * pa[tb][i];
          }
        dl += shfl_xor(dl, 16);
        dl += shfl_xor(dl, 32);  // delta_c = sum p (dO . v)
        const float Lrow = Ls[row];
        const float wc = valid ? fast_exp2((sc - Lrow) * LOG2E) : 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[tb][i] = wc * sa[tb][i] * (pa[tb][i] - dl);  // dx
        f32x4 dqc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) dqc[mb] = zero4();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const FT pf = pk8<T>(sa[2 * ks], sa[2 * ks + 1]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) dqc[mb] = mma16(f.kt[mb][ks], pf, dqc[mb]);
        }
        if (valid) {
          float* dst = accW + row * RS + 4 * (lane >> 4);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            f32x4 cur = *reinterpret_cast<const f32x4*>(dst + 16 * mb);
            cur += scale * dqc[mb];
            *reinterpret_cast<f32x4*>(dst + 16 * mb) = cur;
          }
          if ((lane >> 4) == 0) {
            dsS[row * K + kk] = wc;  // fusion weight, turned into ds once D is known
            dlS[row * K + kk] = dl;
            beta_o[ro * K + kk] = sc - Lrow - (mx * scale + __logf(ls));
            delta_o[ro * K + kk] = dl;
          }
        }
      }
    }
  }
  __syncthreads();
  // chunk part of D = sum over the row's slots of w_c delta_c, in slot order
  for (int r = tid; r < R; r += 256) {
    float a = 0.f;
    for (int kk = 0; kk < K; ++kk) a += dsS[r * K + kk] * dlS[r * K + kk];
    Ds[r] = a;
  }
  __syncthreads();

  // ---------------- window: U1, U2 and its part of D
  {
    const int rbase = w * 16 * CB;
    const int pw_lo = p0 + rbase / G;
    const int pw_hi = min(p0 + (rbase + 16 * CB - 1) / G, N - 1);
    FT qf[CB][KS], df[CB][KS];
    int prow[CB], wsr[CB];
    float Lr[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r = rbase + 16 * cb + (lane & 15);
      const int pos = p0 + r / G, hh = r % G;
      prow[cb] = pos < N ? pos : -1;
      wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
      const int pc = pos < N ? pos : N - 1;
      const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pc;
      Lr[cb] = Ls[r] * LOG2E;
      const T* qs2 = q + ro * DH + 8 * (lane >> 4);
      const T* ds2 = dO + ro * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[cb][ks] = ld8<T>(qs2 + 32 * ks);
        df[cb][ks] = ld8<T>(ds2 + 32 * ks);
      }
    }
    f32x4 u1[MB][CB], u2[MB][CB];
    float dw[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      dw[cb] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        u1[mb][cb] = zero4();
        u2[mb][cb] = zero4();
      }
    }
    if (pw_lo < N) {
      const int kv_lo = n_distant(pw_lo, W, S) * S;
      BwdChunkFrags<T, DH> f;
      for (int kv0 = kv_lo; kv0 <= pw_hi; kv0 += 64) {
        const int nvalid = min(64, N - kv0);
        bwd_load_block<T, DH>(f, kg + (size_t)kv0 * DH, vg + (size_t)kv0 * DH, nvalid, ktg + kv0, Np, lane);
        f32x4 sa[4][CB], pa[4][CB];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            sa[tb][cb] = zero4();
            pa[tb][cb] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              sa[tb][cb] = mma16(f.k[tb][ks], qf[cb][ks], sa[tb][cb]);
              pa[tb][cb] = mma16(f.v[tb][ks], df[cb][ks], pa[tb][cb]);
            }
          }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = kv0 + 16 * tb + 4 * (lane >> 4) + i;
              const bool ok = j <= prow[cb] && j >= wsr[cb];
              const float a = ok ? fast_exp2(fmaf(sa[tb][cb][i], sc2, -Lr[cb])) : 0.f;
              const float adp = a * pa[tb][cb][i];
              dw[cb] += adp;
              sa[tb][cb][i] = a;
              pa[tb][cb][i] = adp;
            }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
              u1[mb][cb] = mma16(f.kt[mb][ks], pk8<T>(pa[2 * ks][cb], pa[2 * ks + 1][cb]), u1[mb][cb]);
              u2[mb][cb] = mma16(f.kt[mb][ks], pk8<T>(sa[2 * ks][cb], sa[2 * ks + 1][cb]), u2[mb][cb]);
            }
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float dsum = dw[cb];
      dsum += shfl_xor(dsum, 16);
      dsum += shfl_xor(dsum, 32);
      const int r = rbase + 16 * cb + (lane & 15);
      const float D = dsum + Ds[r];
      float* dst = accW + r * RS + 4 * (lane >> 4);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x4 cur = *reinterpret_cast<const f32x4*>(dst + 16 * mb);
        cur += scale * (u1[mb][cb] - D * u2[mb][cb]);
        *reinterpret_cast<f32x4*>(dst + 16 * mb) = cur;
      }
      wave_lds_sync();
      if ((lane >> 4) == 0) {
        Ds[r] = D;
        if (prow[cb] >= 0) Dv[((size_t)b * Hq + g * G + r % G) * N + prow[cb]] = D;
      }
    }
  }
  __syncthreads();

  // ---------------- ds_c = w_c (delta_c - D); dq = token part + scale sum_c ds_c kL_c
  // (loads are issued in batches before their values are used: a guarded
  // load per element would wait for each in turn)
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
        if (pos >= N) continue;
        const float wc = dsS[x];
        const float dsv = wc == 0.f ? 0.f : wc * (dl[j] - Ds[r]);
        dsS[x] = dsv;
        ds_o[(((size_t)b * Hq + g * G + r % G) * N + pos) * K + kk] = dsv;
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < R * DH / 4; x += 256) {
    const int r = x / (DH / 4), d4 = 4 * (x - r * (DH / 4));
    const int pos = p0 + r / G, hh = r % G;
    if (pos >= N) continue;
    const int32_t* ti = topk_idx + ((size_t)bg * N + pos) * K;
    f32x4 sur = zero4();
    // the row's chunk ids, then their landmark rows, each batch of eight
    // requested at once
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
    const int a0 = r * RS + d4;
    const f32x4 tok = *reinterpret_cast<const f32x4*>(accT + a0) +
                      *reinterpret_cast<const f32x4*>(accT + R * RS + a0) +
                      *reinterpret_cast<const f32x4*>(accT + 2 * R * RS + a0) +
                      *reinterpret_cast<const f32x4*>(accT + 3 * R * RS + a0);
    const size_t ro = ((size_t)b * Hq + g * G + hh) * N + pos;
    *reinterpret_cast<f32x4*>(dq + ro * DH + d4) = tok + sur;
    if (dqhat != nullptr) *reinterpret_cast<f32x4*>(dqhat + ro * DH + d4) = sur;
  }
}

// --------------------------------------------------------------- dk / dv pass
// One workgroup per 64-token key block. Its rows are the window rows (every
// position whose window covers the block, all heads of the group) and the
// rows that selected the block as a chunk. A wave owns TW 16-token blocks
// and a share of the 32-row groups and keeps dK / dV of its tokens in
// registers; the waves of a token group add their sums at the end.
// dK = dS^T Q and dV = P^T dO contract over rows, so Q and dO are needed with
// the rows as the per-lane k index: the row-major fragments already in
// registers are turned into that layout by a product with the identity
// (exact: every product is x * 1 or x * 0).
// The rows' data are prefetched (list entries two groups ahead; biases,
// deltas, q / dO fragments and u rows one group ahead) so their latency hides
// behind the current group's products.
// dkL_c = scale sum_rows ds q_hat with q_hat = q + W_up u: the q part is one
// more product of the transposed q fragments with ds (hi + lo bf16 halves);
// the u part is added by k_bwd_dklu.
struct DkdvRow {
  int ro;      // query row (b, h, i) of this lane's group row
  int pos;     // position (masking), -1 for padding rows
  float bias;  // raw -lse (window) or beta (chunk)
  float dlt;   // D (window) or delta_c (chunk)
  float dsv;   // ds_c of the slot (chunk rows)
};

template <typename T, int G, int DH>
__global__ __launch_bounds__(256, sizeof(T) == 2 && DH == 64 ? 2 : 1) void k_bwd_dkdv(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dv,
    const int* __restrict__ ioff, const int* __restrict__ ilst, const float* __restrict__ ds_i,
    const float* __restrict__ beta_i, const float* __restrict__ delta_i, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dkL, float* __restrict__ de, int N, int Hkv,
    int K, int W, float scale, int C) {
  typedef typename Frag<T>::type FT;
  constexpr int KS = DH / 32, MB = DH / 16;
  // 16-token blocks per wave: two keep the dK / dV accumulators small enough
  // for two waves per SIMD (all 64 tokens per wave would need one)
  constexpr int TW = 2;
  constexpr int NTG = 4 / TW, WPG = 4 / NTG;  // token groups, waves per token group
  constexpr int MBL = MB / NTG;               // d blocks of the dkL product per token group
  extern __shared__ __align__(16) float red[];  // [2][64][DH]
  __shared__ float redl[DH];
  __shared__ float redd;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int gl = lane >> 4, cl = lane & 15;
  const int tg = w / WPG, wi = w - tg * WPG;
  int blk, bg;
  xcd_block(blk, bg);
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int kv0 = blk * 64;
  const int nvalid = min(64, N - kv0);
  for (int x = tid; x < DH; x += 256) redl[x] = 0.f;
  if (tid == 0) redd = 0.f;

  // the block's K / V rows in LDS (padded pitch: conflict-free fragment
  // reads); they are the B operands of S = Q K^T and dP = dO V^T
  constexpr int KP = DH + 16 / (int)sizeof(T);
  T* ks_l = reinterpret_cast<T*>(red);  // [64][KP]
  T* vs_l = ks_l + 64 * KP;             // [64][KP]
  for (int x = tid; x < 64 * DH / 8; x += 256) {
    const int tok = x / (DH / 8), d8 = 8 * (x - tok * (DH / 8));
    const int tk = tok < nvalid ? tok : 0;
    const size_t o = ((size_t)bg * N + kv0 + tk) * DH + d8;
    *reinterpret_cast<FT*>(ks_l + tok * KP + d8) = ld8<T>(k + o);
    *reinterpret_cast<FT*>(vs_l + tok * KP + d8) = ld8<T>(v + o);
  }
  __syncthreads();
  // identity fragments: I_h[k][col] = (k == 16 h + col)
  FT idf[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float x[8];
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2) x[e2] = (8 * gl + e2 == 16 * h + cl) ? 1.f : 0.f;
    idf[h] = pack8<T>(x);
  }

  const int i_hi = min(N - 1, kv0 + 64 + W - 2);
  const int nw = (i_hi - kv0 + 1) * G;
  const bool chunk = blk < C;
  const int e0 = chunk ? ioff[(size_t)bg * (C + 1) + blk] : 0;
  const int ne = chunk ? ioff[(size_t)bg * (C + 1) + blk + 1] - e0 : 0;
  const int* lst = ilst + (size_t)bg * N * K + e0;
  const int ngw = (nw + 31) / 32, ngt = ngw + (ne * G + 31) / 32;
  const int rowx = lane & 31;  // group row whose data this lane fetches

  // Row data are fetched without branches (out-of-range groups read a valid
  // dummy address) and checked where they are used, so the loads stay in
  // flight behind the current group's products.
  auto fetch_e = [&](int gi) __attribute__((always_inline)) {
    const int rr = 32 * (gi - ngw) + rowx;
    const bool ok = gi >= ngw && rr < ne * G;
    return *(ok ? lst + rr / G : ioff);
  };
  auto fetch_m = [&](int gi, int en) __attribute__((always_inline)) {
    DkdvRow m;
    const bool isw = gi < ngw;
    const int rw = 32 * gi + rowx, rc = 32 * (gi - ngw) + rowx;
    const bool okw = rw < nw, okc = !isw && rc < ne * G;
    const int posw = kv0 + (okw ? rw : 0) / G, hhw = (okw ? rw : 0) % G;
    const int posc = okc ? en >> 6 : 0, kk = okc ? en & 63 : 0, hhc = rowx % G;
    const int pos = isw ? posw : posc, hh = isw ? hhw : hhc;
    m.ro = (b * Hq + g * G + hh) * N + pos;
    m.pos = isw ? (okw ? pos : -1) : (okc ? N : -1);
    const size_t idx = isw ? (size_t)m.ro : (size_t)m.ro * K + kk;
    m.bias = (isw ? lse : beta_i)[idx];
    m.dlt = (isw ? Dv : delta_i)[idx];
    m.dsv = ds_i[isw ? 0 : idx];
    return m;
  };
  auto fetch_q = [&](const DkdvRow& m, FT (&qa)[2][KS], FT (&da)[2][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int ro = __shfl(m.ro, 16 * rb + cl, 64);
      const size_t o = (size_t)ro * DH + 8 * gl;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[rb][ks] = ld8<T>(q + o + 32 * ks);
        da[rb][ks] = ld8<T>(dO + o + 32 * ks);
      }
    }
  };
  // per-wave slots of the current group's row values (bias, delta, pos, ds)
  __shared__ f32x4 mrow_all[4][32];
  f32x4* mrow = mrow_all[w];
  f32x4 dka[TW][MB], dva[TW][MB], dklm[MBL];
#pragma unroll
  for (int tb = 0; tb < TW; ++tb)
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      dka[tb][nb] = zero4();
      dva[tb][nb] = zero4();
    }
#pragma unroll
  for (int nb = 0; nb < MBL; ++nb) dklm[nb] = zero4();
  float dsum = 0.f;
  const float sc2 = scale * LOG2E;

  auto compute = [&](int gi, const DkdvRow& m, const FT (&qa)[2][KS], const FT (&da)[2][KS],
                     auto masked) __attribute__((always_inline)) {
    constexpr bool MSK = decltype(masked)::value;
    const bool isw = gi < ngw;
    // Row values reach the lanes of the D layout (row 16 rb + 4 gl + i)
    // through the wave's LDS slots: plain stores and loads, which (unlike
    // lane shuffles) stay correct when the compiler predicates their uses.
    {
      const bool okr = m.pos >= 0;
      f32x4 mv;
      mv[0] = okr ? (isw ? -m.bias : m.bias) * LOG2E : NEG_INF;
      mv[1] = okr ? m.dlt : 0.f;
      mv[2] = __int_as_float(m.pos);
      mv[3] = okr ? m.dsv : 0.f;
      mrow[rowx] = mv;
      wave_lds_sync();
    }
    float bi[2][4], dl[2][4], dsr[2][4];
    int ps[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 rv = mrow[16 * rb + 4 * gl + i];
        bi[rb][i] = rv[0];
        dl[rb][i] = rv[1];
        ps[rb][i] = __float_as_int(rv[2]);
        dsr[rb][i] = rv[3];
      }
    // per 16-token block: S and dP, then P (a_j) and dS packed as the A
    // operands P^T and dS^T (token 16 (tg TW + tb) + cl)
    FT pA[TW], sA[TW];
#pragma unroll
    for (int tb = 0; tb < TW; ++tb) {
      f32x4 sa[2], pa[2];
      const int trow = (16 * (tg * TW + tb) + cl) * KP + 8 * gl;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        sa[rb] = zero4();
        pa[rb] = zero4();
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FT kf = *reinterpret_cast<const FT*>(ks_l + trow + 32 * ks);
        const FT vf = *reinterpret_cast<const FT*>(vs_l + trow + 32 * ks);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sa[rb] = mma16(qa[rb][ks], kf, sa[rb]);
          pa[rb] = mma16(da[rb][ks], vf, pa[rb]);
        }
      }
      const int tok = 16 * (tg * TW + tb) + cl;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float a = fast_exp2(fmaf(sa[rb][i], sc2, bi[rb][i]));
          if constexpr (MSK) a = (tok < nvalid && kv0 + tok <= ps[rb][i]) ? a : 0.f;
          sa[rb][i] = a;
          pa[rb][i] = a * (pa[rb][i] - dl[rb][i]);
        }
      pA[tb] = pk8<T>(sa[0], sa[1]);
      sA[tb] = pk8<T>(pa[0], pa[1]);
    }
    // ds of the group rows as the first row of an A operand (hi + lo halves)
    FT dsh, dsl;
    const bool dkl_here = !isw;
    if (dkl_here) {
      float hi[8], lo[8];
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) hi[e2] = cl == 0 ? dsr[e2 >> 2][e2 & 3] : 0.f;
      dsh = pack8<T>(hi);
      if constexpr (sizeof(T) == 2) {
        const u16x8 hb = __builtin_bit_cast(u16x8, dsh);
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) lo[e2] = hi[e2] - bf2f(hb[e2]);
        dsl = pack8<T>(lo);
      }
      dsum += (tg == 0 && lane < 32 && m.pos >= 0) ? m.dsv : 0.f;
    }
#pragma unroll
    for (int nb = 0; nb < MB; ++nb) {
      const int ks = nb >> 1, h = nb & 1;
      const FT qT = pk8<T>(mma16(qa[0][ks], idf[h], zero4()), mma16(qa[1][ks], idf[h], zero4()));
      const FT dT = pk8<T>(mma16(da[0][ks], idf[h], zero4()), mma16(da[1][ks], idf[h], zero4()));
#pragma unroll
      for (int tb = 0; tb < TW; ++tb) {
        dva[tb][nb] = mma16(pA[tb], dT, dva[tb][nb]);
        dka[tb][nb] = mma16(sA[tb], qT, dka[tb][nb]);
      }
      if (dkl_here && nb / MBL == tg) {
        dklm[nb % MBL] = mma16(dsh, qT, dklm[nb % MBL]);
        if constexpr (sizeof(T) == 2) dklm[nb % MBL] = mma16(dsl, qT, dklm[nb % MBL]);
      }
    }
  };

  // two register sets take turns: while one group is computed the next
  // group's data load into the other set
  {
    FT qa0[2][KS], da0[2][KS], qa1[2][KS], da1[2][KS];
    int gi = wi;
    int en0 = fetch_e(gi), en1 = fetch_e(gi + WPG);
    DkdvRow m0 = fetch_m(gi, en0), m1;
    fetch_q(m0, qa0, da0);
    auto run = [&](int gc, const DkdvRow& m, const FT (&qa)[2][KS], const FT (&da)[2][KS])
        __attribute__((always_inline)) {
      if (gc < ngw && (32 * gc / G < 63 || nvalid < 64)) compute(gc, m, qa, da, std::true_type());
      else compute(gc, m, qa, da, std::false_type());
    };
    while (gi < ngt) {
      en0 = fetch_e(gi + 2 * WPG);
      m1 = fetch_m(gi + WPG, en1);
      fetch_q(m1, qa1, da1);
      run(gi, m0, qa0, da0);
      gi += WPG;
      if (gi >= ngt) break;
      en1 = fetch_e(gi + 2 * WPG);
      m0 = fetch_m(gi + WPG, en0);
      fetch_q(m0, qa0, da0);
      run(gi, m1, qa1, da1);
      gi += WPG;
    }
  }

  // ---- reductions: dK / dV by the waves of each token group in turn
  for (int turn = 0; turn < WPG; ++turn) {
    __syncthreads();
    if (wi == turn) {
#pragma unroll
      for (int tb = 0; tb < TW; ++tb)
#pragma unroll
        for (int nb = 0; nb < MB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * (tg * TW + tb) + 4 * gl + i;
            const int x = tok * DH + 16 * nb + cl;
            const float a = turn ? red[x] : 0.f;
            const float c = turn ? red[64 * DH + x] : 0.f;
            red[x] = a + dka[tb][nb][i];
            red[64 * DH + x] = c + dva[tb][nb][i];
          }
    }
  }
  if (chunk) {
    if (lane < 16) {
#pragma unroll
      for (int nb = 0; nb < MBL; ++nb) atomicAdd(&redl[16 * (tg * MBL + nb) + cl], dklm[nb][0]);
    }
    if (tg == 0) {
      float s2 = dsum;
#pragma unroll
      for (int m2 = 32; m2 >= 1; m2 >>= 1) s2 += __shfl_xor(s2, m2, 64);
      if (lane == 0) atomicAdd(&redd, s2);
    }
  }
  __syncthreads();
  for (int x = tid; x < 64 * DH; x += 256) {
    const int tok = x / DH;
    if (tok < nvalid) {
      const size_t o = ((size_t)bg * N + kv0 + tok) * DH + (x - tok * DH);
      dk[o] = red[x] * scale;
      dv[o] = red[64 * DH + x];
    }
  }
  if (chunk) {
    for (int x = tid; x < DH; x += 256) dkL[((size_t)bg * C + blk) * DH + x] = redl[x] * scale;
    if (tid == 0) de[(size_t)bg * C + blk] = redd;
  }
}

// Q-Cal part of the landmark gradient: dkL_c += scale sum_h W_up[h] U_h with
// U_h = sum over the rows of head h that selected chunk c of ds u_row. One
// workgroup per chunk. R / 4 adjacent lanes share a row (lane q loads u
// elements 4q .. 4q + 3), so one wave load covers whole 128-byte rows rather
// than one line per lane; a lane's rows are entries rs, rs + 256 / (R / 4),
// ... (rs its row slot, so its head rs % G is fixed). Eight rows per lane are
// in flight, with the next eight rows' list entries. The lanes of a head and
// quad are summed across the wave's row slots, then across the waves in LDS.
template <typename T, int R>
__global__ __launch_bounds__(256) void k_bwd_dklu(const int* __restrict__ ioff,
                                                  const int* __restrict__ ilst,
                                                  const float* __restrict__ ds_i,
                                                  const float* __restrict__ u,
                                                  const T* __restrict__ W_up,
                                                  float* __restrict__ dkL, int N, int Hkv, int G,
                                                  int K, int C, int d, float scale) {
  constexpr int LPR = R / 4, RPI = 256 / LPR, RU = 8;
  __shared__ f32x4 part[4][64];
  __shared__ float us[256];  // [G][R]
  int c, bg;
  xcd_block(c, bg);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = bg / Hkv, g = bg - b * Hkv, Hq = Hkv * G;
  const int e0 = ioff[(size_t)bg * (C + 1) + c];
  const int nrow = (ioff[(size_t)bg * (C + 1) + c + 1] - e0) * G;
  const int* lst = ilst + (size_t)bg * N * K + e0;
  const int rs = tid / LPR, q = tid - rs * LPR;
  const int h = g * G + rs % G;
  const float* ub = u + (size_t)b * N * Hq * R + (size_t)h * R + 4 * q;  // + pos Hq R
  const float* db = ds_i + (size_t)(b * Hq + h) * N * K;                // + pos K + slot
  f32x4 acc = zero4();
  if (nrow > 0) {
    int en[RU];
#pragma unroll
    for (int t = 0; t < RU; ++t) en[t] = lst[min(rs + RPI * t, nrow - 1) / G];
    for (int x0 = rs; x0 < nrow; x0 += RPI * RU) {
      float dsv[RU];
      f32x4 uv[RU];
#pragma unroll
      for (int t = 0; t < RU; ++t) {
        const int pos = en[t] >> 6, kk = en[t] & 63;
        const float dv = db[(size_t)pos * K + kk];
        dsv[t] = x0 + RPI * t < nrow ? dv : 0.f;
        uv[t] = *reinterpret_cast<const f32x4*>(ub + (size_t)pos * Hq * R);
      }
#pragma unroll
      for (int t = 0; t < RU; ++t) en[t] = lst[min(x0 + RPI * (RU + t), nrow - 1) / G];
#pragma unroll
      for (int t = 0; t < RU; ++t) acc += dsv[t] * uv[t];
    }
  }
  // sum over the wave's row slots of one head: lanes l, l ^ m for m >= LPR G
#pragma unroll
  for (int m = 32; m >= LPR; m >>= 1) {
    if (m < LPR * G) break;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) acc[e2] += __shfl_xor(acc[e2], m, 64);
  }
  if (lane < LPR * G) part[w][lane] = acc;  // lane = head * LPR + quad
  __syncthreads();
  if (tid < G * R) {
    const int h2 = tid / R, j = tid - h2 * R;
    const int l = h2 * LPR + j / 4;
    us[tid] = part[0][l][j & 3] + part[1][l][j & 3] + part[2][l][j & 3] + part[3][l][j & 3];
  }
  __syncthreads();
  for (int dd = tid; dd < d; dd += 256) {
    float val = 0.f;
    for (int h2 = 0; h2 < G; ++h2) {
      const T* wr = W_up + ((size_t)(g * G + h2) * d + dd) * R;
#pragma unroll 8
      for (int jj = 0; jj < R; ++jj) val = fmaf(to_f<T>(wr[jj]), us[h2 * R + jj], val);
    }
    dkL[((size_t)bg * C + c) * d + dd] += val * scale;
  }
}

// --------------------------------------------------------------- host side
namespace {
struct BwdWs {
  float *qhat, *u, *Dv, *sT, *ds, *beta, *delta, *dqhat, *du, *gwork;
  int *off, *lst;
  InvIndex ix;
  void* kt;
  const void* W_up;
  int Np, ns;
};
size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
// dW_down[h] += sum_i du[b, i, h, :] (x) h[b, i, :]: all heads and all batch
// elements in one product, rows (h, j) of du^T [Hq r x B N] times h [B N x D]
GemmArgs dwdown_args(const Dims& p, float* dW_down) {
  GemmArgs g;
  const long Hr = (long)p.Hq * p.r;
  g.M = (int)Hr; g.N = p.D; g.K = p.B * p.N;
  g.akm = true; g.bkm = false;
  g.lda = Hr; g.ldb = p.D; g.ldc = p.D;
  g.C = dW_down;
  // split K so the launch holds ~2048 64x64 tiles (atomic split-K path)
  const long tiles = (long)((Hr + 63) / 64) * ((p.D + 63) / 64);
  g.splits = (int)std::max(1L, std::min((long)(g.K / 256), (2048 + tiles - 1) / tiles));
  g.accumulate = true;
  return g;
}
size_t carve(const Dims& p, void* base, BwdWs* w) {
  char* c = static_cast<char*>(base);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    void* ptr = c ? c + o : nullptr;
    o += up256(bytes);
    return ptr;
  };
  const size_t rows = (size_t)p.B * p.Hq * p.N;
  const size_t bg = (size_t)p.B * p.Hkv;
  const bool qc = p.r > 0;
  w->qhat = (float*)take(qc ? rows * p.d * 4 : 0);
  w->u = (float*)take(qc ? (size_t)p.B * p.N * p.Hq * p.r * 4 : 0);
  w->Dv = (float*)take(rows * 4);
  w->sT = (float*)take(rows * p.K * 4);
  w->ds = (float*)take(rows * p.K * 4);
  w->beta = (float*)take(rows * p.K * 4);
  w->delta = (float*)take(rows * p.K * 4);
  w->dqhat = (float*)take(qc ? rows * p.d * 4 : 0);
  w->du = (float*)take(qc ? (size_t)p.B * p.N * p.Hq * p.r * 4 : 0);
  w->gwork = (float*)take(qc ? gemm_work_bytes(dwdown_args(p, nullptr)) : 0);
  {
    InvIndex ix;
    void* ib = take(inv_index_carve(p, nullptr, &ix));
    inv_index_carve(p, ib, &ix);
    w->ix = ix;
    w->off = ix.off;
    w->lst = ix.lst;
  }
  w->Np = (p.N + 63) / 64 * 64;
  w->kt = take(bg * (size_t)p.d * w->Np * (p.dtype == 1 ? 2 : 4));
  return o;
}

template <typename T, int G, int DH, int CB>
size_t dq_lds(const Dims& p) {
  constexpr int R = 64 * CB, TP = R / G;
  size_t NE = 1;
  while (NE < (size_t)TP * p.K) NE <<= 1;
  if (NE > 4096) return (size_t)-1;  // entry ids take 12 bits of the sort keys
  size_t s = sizeof(float) * (4 * (size_t)R * (DH + 4) + 2 * R + 2 * (size_t)R * p.K);
  s += sizeof(int) * (4 * NE + 1) + sizeof(uint16_t) * NE;
  return ((s + 15) & ~(size_t)15) + 64;
}

// row blocks per wave of the dq pass: two when the LDS budget allows
template <typename T, int G, int DH>
int dq_cb(const Dims& p) {
  if (sizeof(T) == 2 && dq_lds<T, G, DH, 2>(p) <= 160 * 1024) return 2;
  return 1;
}

template <typename T>
size_t dq_lds_t(const Dims& p) {
  switch (p.G * 1000 + p.d) {
    case 1064: return dq_cb<T, 1, 64>(p) == 2 ? dq_lds<T, 1, 64, 2>(p) : dq_lds<T, 1, 64, 1>(p);
    case 1128: return dq_cb<T, 1, 128>(p) == 2 ? dq_lds<T, 1, 128, 2>(p) : dq_lds<T, 1, 128, 1>(p);
    case 2064: return dq_cb<T, 2, 64>(p) == 2 ? dq_lds<T, 2, 64, 2>(p) : dq_lds<T, 2, 64, 1>(p);
    case 2128: return dq_cb<T, 2, 128>(p) == 2 ? dq_lds<T, 2, 128, 2>(p) : dq_lds<T, 2, 128, 1>(p);
    case 4064: return dq_cb<T, 4, 64>(p) == 2 ? dq_lds<T, 4, 64, 2>(p) : dq_lds<T, 4, 64, 1>(p);
    case 4128: return dq_cb<T, 4, 128>(p) == 2 ? dq_lds<T, 4, 128, 2>(p) : dq_lds<T, 4, 128, 1>(p);
    default: return (size_t)-1;
  }
}

size_t dq_lds_bytes(const Dims& p) { return p.dtype == 1 ? dq_lds_t<uint16_t>(p) : dq_lds_t<float>(p); }

size_t dkdv_lds(const Dims& p) {
  const size_t el = p.dtype == 1 ? 2 : 4;
  return std::max(2 * 64 * (size_t)p.d * sizeof(float), 2 * 64 * ((size_t)p.d * el + 16));
}

unsigned grid1(size_t n) { return (unsigned)std::min<size_t>((n + 255) / 256, 65535 * 4); }
}  // namespace

size_t bwd_workspace(const Dims& p) {
  if (dq_lds_bytes(p) > 160 * 1024 || dkdv_lds(p) + 1024 > 160 * 1024) return (size_t)-1;
  if ((size_t)p.N * p.K >= (1u << 31)) return (size_t)-1;
  if (!inv_index_ok(p)) return (size_t)-1;
  BwdWs w;
  return carve(p, nullptr, &w);
}

template <typename T, typename QT, int G, int DH>
static hipError_t bwd_go(const Dims& p, const void* q, const void* qsrc, const void* k,
                         const void* v, const void* kL, const void* e, const void* o,
                         const float* lse, const int32_t* topk_idx, const void* dO, float* dq,
                         float* dk, float* dv, float* dkL, float* de, BwdWs& w, hipStream_t st) {
  const size_t rows = (size_t)p.B * p.Hq * p.N;
  const size_t bg = (size_t)p.B * p.Hkv;
  hipError_t err;
  hipLaunchKernelGGL((k_bwd_prep<T, QT, DH>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, st,
                     (const QT*)qsrc, (const T*)kL, (const T*)e, topk_idx, w.sT, (long)rows, p.N,
                     p.Hq, p.Hkv, G, p.C, p.K, p.scale);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // inverse index (deterministic: each chunk's rows in ascending position order)
  if ((err = launch_inv_index(p, topk_idx, w.ix, st)) != hipSuccess) return err;
  // dq pass (K^T copy first)
  {
    hipLaunchKernelGGL((k_vt_perm<T, DH>), dim3(w.Np / 64, (unsigned)bg), dim3(256), 0, st,
                       (const T*)k, (T*)w.kt, p.N, w.Np);
    auto go = [&](auto cbc) -> hipError_t {
      constexpr int CBv = decltype(cbc)::value;
      constexpr int TP = 64 * CBv / G;
      const int ntiles = (p.N + TP - 1) / TP;
      const size_t lds = dq_lds<T, G, DH, CBv>(p);
      auto kern = k_bwd_dq<T, G, DH, CBv>;
      hipError_t e2 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e2 != hipSuccess) return e2;
      hipLaunchKernelGGL(kern, dim3(ntiles, (unsigned)bg), dim3(256), lds, st, (const T*)q,
                         (const T*)k, (const T*)v, (const T*)w.kt, w.Np, (const T*)dO,
                         (const T*)kL, topk_idx, w.sT, lse, w.Dv, dq, w.dqhat, w.ds, w.beta,
                         w.delta, p.N, p.Hkv, p.K, p.W, p.S, p.scale, ntiles, p.C);
      return hipGetLastError();
    };
    // the shared-tile kernel reads the ids as 16-byte vectors
    if (bwd_dq_shared_ok(p) && (reinterpret_cast<uintptr_t>(topk_idx) & 15) == 0)
      err = launch_bwd_dq_shared(p, q, k, v, w.kt, w.Np, dO, kL, topk_idx, w.sT, lse, w.Dv, dq,
                                 w.dqhat, w.ds, w.beta, w.delta, st);
    else
      err = dq_cb<T, G, DH>(p) == 2 ? go(std::integral_constant<int, 2>()) : go(std::integral_constant<int, 1>());
    if (err != hipSuccess) return err;
  }
  // dk / dv pass
  {
    const int nblk = (p.N + 63) / 64;
    const size_t lds = dkdv_lds(p);
    auto kern = k_bwd_dkdv<T, G, DH>;
    if ((err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
      return err;
    hipLaunchKernelGGL(kern, dim3(nblk, (unsigned)bg), dim3(256), lds, st, (const T*)q, (const T*)k,
                       (const T*)v, (const T*)dO, lse, w.Dv, w.off, w.lst, w.ds, w.beta, w.delta,
                       dk, dv, dkL, de, p.N, p.Hkv, p.K, p.W, p.scale, p.C);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (p.r > 0 && p.C > 0) {
    auto dklu = p.r == 16 ? k_bwd_dklu<T, 16> : p.r == 32 ? k_bwd_dklu<T, 32> : k_bwd_dklu<T, 64>;
    hipLaunchKernelGGL(dklu, dim3(p.C, (unsigned)bg), dim3(256), 0, st, w.off, w.lst, w.ds,
                       (const float*)w.u, (const T*)w.W_up, dkL, p.N, p.Hkv, G, p.K, p.C, p.d,
                       p.scale);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

template <typename T, typename QT, int G>
static hipError_t bwd_d(const Dims& p, const void* q, const void* qs, const void* k, const void* v,
                        const void* kL, const void* e, const void* o, const float* lse,
                        const int32_t* idx, const void* dO, float* dq, float* dk, float* dv,
                        float* dkL, float* de, BwdWs& w, hipStream_t st) {
  if (p.d == 64) return bwd_go<T, QT, G, 64>(p, q, qs, k, v, kL, e, o, lse, idx, dO, dq, dk, dv, dkL, de, w, st);
  return bwd_go<T, QT, G, 128>(p, q, qs, k, v, kL, e, o, lse, idx, dO, dq, dk, dv, dkL, de, w, st);
}

template <typename T, typename QT>
static hipError_t bwd_g(const Dims& p, const void* q, const void* qs, const void* k, const void* v,
                        const void* kL, const void* e, const void* o, const float* lse,
                        const int32_t* idx, const void* dO, float* dq, float* dk, float* dv,
                        float* dkL, float* de, BwdWs& w, hipStream_t st) {
  switch (p.G) {
    case 1: return bwd_d<T, QT, 1>(p, q, qs, k, v, kL, e, o, lse, idx, dO, dq, dk, dv, dkL, de, w, st);
    case 2: return bwd_d<T, QT, 2>(p, q, qs, k, v, kL, e, o, lse, idx, dO, dq, dk, dv, dkL, de, w, st);
    case 4: return bwd_d<T, QT, 4>(p, q, qs, k, v, kL, e, o, lse, idx, dO, dq, dk, dv, dkL, de, w, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const Dims& p, const void* q, const void* k, const void* v, const void* kL,
                      const void* e, const void* h, const void* W_down, const void* W_up,
                      const void* o, const float* lse, const int32_t* topk_idx, const void* dO,
                      float* dq, float* dk, float* dv, float* dkL, float* de, float* dW_down,
                      float* dW_up, float* dh, void* ws, hipStream_t st) {
  BwdWs w;
  carve(p, ws, &w);
  w.W_up = W_up;
  const bool qc = p.r > 0;
  hipError_t err;
  if (qc) {
    if ((err = launch_qcal(p, p.N, q, h, W_down, W_up, w.qhat, w.u, st)) != hipSuccess) return err;
  } else {
    w.dqhat = nullptr;
  }
  if (p.dtype == 1) {
    err = qc ? bwd_g<uint16_t, float>(p, q, w.qhat, k, v, kL, e, o, lse, topk_idx, dO, dq, dk, dv, dkL, de, w, st)
             : bwd_g<uint16_t, uint16_t>(p, q, q, k, v, kL, e, o, lse, topk_idx, dO, dq, dk, dv, dkL, de, w, st);
  } else {
    err = bwd_g<float, float>(p, q, qc ? (const void*)w.qhat : q, k, v, kL, e, o, lse, topk_idx, dO,
                              dq, dk, dv, dkL, de, w, st);
  }
  if (err != hipSuccess || !qc) return err;
  // ---- Q-Cal backward
  const long Hr = (long)p.Hq * p.r;
  const long NHr = (long)p.N * Hr;
  const int dt = p.dtype == 1 ? 1 : 0;
  // du[b, i, h, :] = W_up[h]^T dq_hat[b, h, i, :]
  {
    GemmArgs g;
    g.M = p.N; g.N = p.r; g.K = p.d;
    g.akm = false; g.bkm = false;
    g.lda = p.d; g.ldb = p.r; g.ldc = Hr;
    g.n1 = p.B; g.n2 = p.Hq;
    g.sA1 = (long)p.Hq * p.N * p.d; g.sA2 = (long)p.N * p.d;
    g.sB1 = 0; g.sB2 = (long)p.d * p.r;
    g.sC1 = NHr; g.sC2 = p.r;
    g.C = w.du;
    if ((err = gemm(g, w.dqhat, 0, W_up, dt, st)) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(k_fill_f32, dim3(grid1((size_t)Hr * p.D)), dim3(256), 0, st, dW_down, (size_t)Hr * p.D, 0.f);
  hipLaunchKernelGGL(k_fill_f32, dim3(grid1((size_t)p.Hq * p.d * p.r)), dim3(256), 0, st, dW_up, (size_t)p.Hq * p.d * p.r, 0.f);
  // dW_up[h] += sum_i dq_hat[b, h, i, :] (x) u[b, i, h, :]
  {
    GemmArgs g;
    g.M = p.d; g.N = p.r; g.K = p.N;
    g.akm = true; g.bkm = false;
    g.lda = p.d; g.ldb = Hr; g.ldc = p.r;
    g.n1 = p.B; g.n2 = p.Hq;
    g.sA1 = (long)p.Hq * p.N * p.d; g.sA2 = (long)p.N * p.d;
    g.sB1 = NHr; g.sB2 = p.r;
    g.sC1 = 0; g.sC2 = (long)p.d * p.r;
    g.C = dW_up;
    g.splits = std::max(1, p.N / 1024);
    g.accumulate = true;
    if ((err = gemm(g, w.dqhat, 0, w.u, 0, st)) != hipSuccess) return err;
  }
  {
    GemmArgs g = dwdown_args(p, dW_down);
    g.work = w.gwork;
    if ((err = gemm(g, w.du, 0, h, dt, st)) != hipSuccess) return err;
  }
  // dh[b, i, :] = sum_{h, j} du[b, i, h, j] W_down[h, j, :]
  if (dh != nullptr) {
    GemmArgs g;
    g.M = p.N; g.N = p.D; g.K = (int)Hr;
    g.akm = false; g.bkm = false;
    g.lda = Hr; g.ldb = p.D; g.ldc = p.D;
    g.n1 = p.B; g.n2 = 1;
    g.sA1 = NHr; g.sB1 = 0; g.sC1 = (long)p.N * p.D;
    g.C = dh;
    if ((err = gemm(g, w.du, 0, W_down, dt, st)) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace hils
