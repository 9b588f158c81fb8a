// HiLS prefill forward, bucketed strategy: for tiles whose selections are
// spread over many chunks (few rows per chunk), the chunk phase buckets the
// tile's (position, slot) selections by chunk and lets waves take chunks
// dynamically, so each chunk's K / V^T is read once per tile and its rows are
// packed densely into MFMA row blocks.
//
// Paper: same computation as the shared-block strategy in attn_fwd.hip
// (window attention, per-chunk attention, fusion by the selection scores).
//
// Tile: R = 64 * CB rows = TP positions x G heads of one (batch, KV head),
// four waves.
//   Window phase: wave w runs a banded flash attention over its 16*CB rows
//     with K and V^T fragments loaded straight from global memory (the next
//     key block prefetched into a second register set). The fusion
//     normaliser L follows from lse_W and the log-sum-exp of the selected
//     scores, and exp(lse_W - L) O_W seeds the row accumulators.
//   Chunk phase: selections are bucketed by chunk (counting sort in LDS);
//     waves take chunks dynamically and add exp(s_c - L) O_c for each row
//     block into a per-wave fp32 accumulator copy in LDS (plain
//     read-modify-write; the four copies are summed at the end).
#include "hils_common.h"
#include "hils_internal.h"

#include <algorithm>
#include <type_traits>

namespace hils {

template <typename T, int DH>
struct BlockFrags {
  typename Frag<T>::type k[4][DH / 32];  // A operand of S^T: K rows (tokens)
  typename Frag<T>::type v[DH / 16][2];  // A operand of O^T: V^T rows (dims)
};

// K rows kbase + 16*tb + lane%16 (clamped below nvalid) and the permuted V^T
// columns vtbase + 32*ks + 8*(lane/16) of dims 16*mb + lane%16.
template <typename T, int DH>
__device__ __forceinline__ void load_block(BlockFrags<T, DH>& f, const T* __restrict__ kbase, int nvalid,
                                           const T* __restrict__ vtbase, int Np, int lane) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    int tok = 16 * tb + (lane & 15);
    tok = tok < nvalid ? tok : 0;
    const T* src = kbase + (size_t)tok * DH + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) f.k[tb][ks] = ld8<T>(src + 32 * ks);
  }
#pragma unroll
  for (int mb = 0; mb < DH / 16; ++mb) {
    const T* src = vtbase + (size_t)(16 * mb + (lane & 15)) * Np + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) f.v[mb][ks] = ld8<T>(src + 32 * ks);
  }
}

template <typename T, int DH>
struct RowFrags {
  typename Frag<T>::type q[DH / 32];
  float s;     // fusion score of the row's chunk
  int row;     // tile row
  bool valid;
};

template <typename T, int G, int DH, int CB>
__global__ __launch_bounds__(256) void k_attn_fwd_sparse(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ vt,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_score,
    const float* __restrict__ sel_lse, T* __restrict__ o, float* __restrict__ lse, int N, int Np,
    int Hkv, int K, int W, int S, float scale, int ntiles, int C) {
  typedef typename Frag<T>::type FT;
  constexpr int R = 64 * CB;        // rows per tile
  constexpr int TP = R / G;         // positions per tile
  constexpr int KS = DH / 32;
  constexpr int MB = DH / 16;
  constexpr int RS = DH + 4;        // accumulator row stride (floats)
  constexpr int EPT = TP * 32 / 256;  // max entries per thread (K <= 32)
  constexpr bool PF = DH == 64;     // double-buffered prefetch (register budget)

  extern __shared__ __align__(16) unsigned char smem[];
  // one accumulator copy per wave: waves add their chunk contributions to
  // their own copy with plain read-modify-write (no LDS atomics), and the
  // copies are summed when the tile is written out
  float* accT = reinterpret_cast<float*>(smem);          // [4][R][RS]
  float* Ls = accT + 4 * R * RS;                         // [R]
  int* off = reinterpret_cast<int*>(Ls + R);             // [C + 1] counts -> offsets
  int* nzl = off + C + 1;                                // [C] ranks -> nonempty chunk ids
  uint16_t* ent = reinterpret_cast<uint16_t*>(nzl + C);  // [TP*K]
  __shared__ int wsum[4];
  __shared__ int ctr;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int tx, bg;
  xcd_block(tx, bg);
  const int tile = ntiles - 1 - tx;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int Hq = Hkv * G;
  const int p0 = tile * TP;
  const int plast = min(p0 + TP - 1, N - 1);
  const int ndmax = n_distant(plast, W, S);  // chunks any row of the tile can select
  const T* kg = k + (size_t)bg * N * DH;
  const T* vtg = vt + (size_t)bg * DH * Np;
  float* accW = accT + w * R * RS;  // this wave's accumulator copy

  // ------------------------------------------------ bucket selections by chunk
  for (int x = tid; x <= ndmax; x += 256) off[x] = 0;
  if (tid == 0) ctr = 0;
  for (int x = tid; x < R * RS; x += 256) reinterpret_cast<f32x4*>(accT)[x] = zero4();
  __syncthreads();
  int my_c[EPT], my_r[EPT];
  const int E = TP * K;
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
    my_r[j] = 0;
    const bool ok = x < E && p0 + x / K < N && c >= 0 && c < ndmax;
    my_c[j] = ok ? c : -1;
    if (ok) my_r[j] = atomicAdd(&off[c], 1);
  }
  __syncthreads();
  for (int x = tid; x < ndmax; x += 256) nzl[x] = off[x] > 0 ? 1 : 0;
  __syncthreads();
  const int Etot = block_excl_scan(off, ndmax, wsum);
  const int NZ = block_excl_scan(nzl, ndmax, wsum);
  if (tid == 0) off[ndmax] = Etot;
  __syncthreads();
  // ranks -> list of nonempty chunk ids (a rank never exceeds its chunk id, so
  // reading a block of ranks before writing keeps later ranks intact)
  for (int base = 0; base < ndmax; base += 256) {
    const int x = base + tid;
    const int rk = (x < ndmax && off[x + 1] > off[x]) ? nzl[x] : -1;
    __syncthreads();
    if (rk >= 0) nzl[rk] = x;
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int c = my_c[j];
    if (c >= 0) {
      const int x = tid + 256 * j;
      const int pl = x / K, kk = x - pl * K;
      ent[off[c] + my_r[j]] = (uint16_t)((pl << 6) | kk);
    }
  }

  // ------------------------------------------------ window phase
  {
    const int rbase = w * 16 * CB;                 // first tile row of this wave
    const int pw_lo = p0 + rbase / G;
    const int pw_hi = min(p0 + (rbase + 16 * CB - 1) / G, N - 1);
    FT qf[CB][KS];
    int prow[CB], wsr[CB];
    float lsel[CB];  // log-sum-exp of the row's selected chunk scores
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r = rbase + 16 * cb + (lane & 15);
      const int pos = p0 + r / G, hh = r % G;
      prow[cb] = pos < N ? pos : -1;
      wsr[cb] = pos < N ? n_distant(pos, W, S) * S : 0;
      const int pc = pos < N ? pos : N - 1;
      lsel[cb] = sel_lse[((size_t)b * Hq + g * G + hh) * N + pc];
      const T* src = q + (((size_t)b * Hq + g * G + hh) * N + pc) * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[cb][ks] = ld8<T>(src + 32 * ks);
    }
    float m[CB], lsum[CB];
    f32x4 oacc[MB][CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      m[cb] = NEG_INF;
      lsum[cb] = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] = zero4();
    }
    // rows of this wave whose window does not cover a whole block need masks;
    // a block strictly inside every row's window is processed without them
    int minpos = 1 << 30, maxws = 0;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      minpos = min(minpos, prow[cb] >= 0 ? prow[cb] : -1);
      maxws = max(maxws, wsr[cb]);
    }
#pragma unroll
    for (int m2 = 1; m2 < 16; m2 <<= 1) {
      minpos = min(minpos, __shfl_xor(minpos, m2, 64));
      maxws = max(maxws, __shfl_xor(maxws, m2, 64));
    }
    const float sc2 = scale * LOG2E;  // logits in base 2
    auto compute = [&](const BlockFrags<T, DH>& f, int kv0, auto masked) __attribute__((always_inline)) {
      f32x4 sacc[4][CB];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          sacc[tb][cb] = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) sacc[tb][cb] = mma16(f.k[tb][ks], qf[cb][ks], sacc[tb][cb]);
        }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        float bmax = NEG_INF;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = sacc[tb][cb][i] * sc2;
            if constexpr (decltype(masked)::value) {
              const int j = kv0 + 16 * tb + 4 * (lane >> 4) + i;
              x = (j <= prow[cb] && j >= wsr[cb]) ? x : NEG_INF;
            }
            sacc[tb][cb][i] = x;
            bmax = fmaxf(bmax, x);
          }
        bmax = fmaxf(bmax, shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, shfl_xor(bmax, 32));
        const float mnew = fmaxf(m[cb], bmax);
        const float mref = mnew == NEG_INF ? 0.f : mnew;
        const float alpha = fast_exp2(m[cb] - mref);
        float ps = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = fast_exp2(sacc[tb][cb][i] - mref);
            sacc[tb][cb][i] = pv;
            ps += pv;
          }
        lsum[cb] = lsum[cb] * alpha + ps;
        m[cb] = mnew;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb][cb] *= alpha;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        FT pf[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) pf[cb] = pk8<T>(sacc[2 * ks][cb], sacc[2 * ks + 1][cb]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) oacc[mb][cb] = mma16(f.v[mb][ks], pf[cb], oacc[mb][cb]);
      }
    };
    auto run = [&](const BlockFrags<T, DH>& f, int kv0) __attribute__((always_inline)) {
      const bool clean = minpos >= 0 && kv0 >= maxws && kv0 + 63 <= minpos;
      if (clean)
        compute(f, kv0, std::false_type());
      else
        compute(f, kv0, std::true_type());
    };
    if (pw_lo < N && !PF) {
      const int kv_lo = n_distant(pw_lo, W, S) * S;
      BlockFrags<T, DH> fa;
      for (int kv0 = kv_lo; kv0 <= pw_hi; kv0 += 64) {
        load_block<T, DH>(fa, kg + (size_t)kv0 * DH, min(64, N - kv0), vtg + kv0, Np, lane);
        run(fa, kv0);
      }
    } else if (pw_lo < N) {
      const int kv_lo = n_distant(pw_lo, W, S) * S;
      BlockFrags<T, DH> fa, fb;
      load_block<T, DH>(fa, kg + (size_t)kv_lo * DH, min(64, N - kv_lo), vtg + kv_lo, Np, lane);
      for (int kv0 = kv_lo; kv0 <= pw_hi; kv0 += 128) {
        const int k1 = kv0 + 64;
        if (k1 <= pw_hi) load_block<T, DH>(fb, kg + (size_t)k1 * DH, min(64, N - k1), vtg + k1, Np, lane);
        run(fa, kv0);
        if (k1 > pw_hi) break;
        const int k2 = kv0 + 128;
        if (k2 <= pw_hi) load_block<T, DH>(fa, kg + (size_t)k2 * DH, min(64, N - k2), vtg + k2, Np, lane);
        run(fb, k1);
      }
    }
    // window log-sum-exp, fusion normaliser, window contribution
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float ls = lsum[cb];
      ls += shfl_xor(ls, 16);
      ls += shfl_xor(ls, 32);
      const int r = rbase + 16 * cb + (lane & 15);
      const int hh = r % G;
      const int pc = prow[cb] >= 0 ? prow[cb] : N - 1;
      const size_t rowoff = ((size_t)b * Hq + g * G + hh) * N + pc;
      const float lW = (m[cb] + __log2f(ls)) * LN2;  // natural log-sum-exp of the window
      // L = log(exp(lW) + sum over the selected chunks of exp(s_c))
      const float mx = fmaxf(lW, lsel[cb]);
      const bool live = prow[cb] >= 0;
      const float L = live ? mx + __logf(__expf(lW - mx) + __expf(lsel[cb] - mx)) : 0.f;
      const float coef = live ? fast_exp2(m[cb] - L * LOG2E) : 0.f;
      if ((lane >> 4) == 0) {
        Ls[r] = L;
        if (live) lse[rowoff] = L;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        *reinterpret_cast<f32x4*>(accW + r * RS + 16 * mb + 4 * (lane >> 4)) = oacc[mb][cb] * coef;
    }
  }
  __syncthreads();

  // ------------------------------------------------ chunk phase
  {
    auto grab = [&]() __attribute__((always_inline)) {
      int it = 0;
      if (lane == 0) it = atomicAdd(&ctr, 1);
      return __shfl(it, 0, 64);
    };
    // row fragments of row block cbk of a chunk whose entries are e0 .. e0 + n
    auto load_rows = [&](RowFrags<T, DH>& rf, int e0, int n, int cbk) __attribute__((always_inline)) {
      const int rr = 16 * cbk + (lane & 15);
      rf.valid = rr < n * G;
      const int ei = (rf.valid ? rr : 0) / G, hh = (rf.valid ? rr : 0) % G;
      const int en = ent[e0 + ei];
      const int pl = en >> 6, kk = en & 63;
      rf.row = pl * G + hh;
      const size_t rowoff = ((size_t)b * Hq + g * G + hh) * N + p0 + pl;
      const T* src = q + rowoff * DH + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) rf.q[ks] = ld8<T>(src + 32 * ks);
      rf.s = topk_score[rowoff * K + kk];
    };
    auto process_rows = [&](const BlockFrags<T, DH>& f, const RowFrags<T, DH>& rf) __attribute__((always_inline)) {
      f32x4 sacc[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        sacc[tb] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc[tb] = mma16(f.k[tb][ks], rf.q[ks], sacc[tb]);
      }
      const float sc2 = scale * LOG2E;
      float mx = NEG_INF;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[tb][i]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mref = mx * sc2;
      float ps = 0.f;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(fmaf(sacc[tb][i], sc2, -mref));
          sacc[tb][i] = pv;
          ps += pv;
        }
      ps += shfl_xor(ps, 16);
      ps += shfl_xor(ps, 32);
      f32x4 oc[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oc[mb] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const FT pf = pk8<T>(sacc[2 * ks], sacc[2 * ks + 1]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oc[mb] = mma16(f.v[mb][ks], pf, oc[mb]);
      }
      if (rf.valid) {
        const float alpha = fast_exp2((rf.s - Ls[rf.row]) * LOG2E) / ps;
        float* dst = accW + rf.row * RS + 4 * (lane >> 4);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4 cur = *reinterpret_cast<const f32x4*>(dst + 16 * mb);
          cur += alpha * oc[mb];
          *reinterpret_cast<f32x4*>(dst + 16 * mb) = cur;
        }
      }
    };
    auto process_chunk = [&](const BlockFrags<T, DH>& f, RowFrags<T, DH>& r0, int c) __attribute__((always_inline)) {
      const int e0 = off[c], n = off[c + 1] - e0;
      const int nb = (n * G + 15) / 16;
      RowFrags<T, DH> r1;
      for (int cbk = 0; cbk < nb; cbk += 2) {
        if (cbk + 1 < nb) load_rows(r1, e0, n, cbk + 1);
        process_rows(f, r0);
        if (cbk + 1 >= nb) break;
        if (cbk + 2 < nb) load_rows(r0, e0, n, cbk + 2);
        process_rows(f, r1);
      }
    };
    auto load_chunk = [&](BlockFrags<T, DH>& f, RowFrags<T, DH>& r0, int c) __attribute__((always_inline)) {
      load_block<T, DH>(f, kg + (size_t)c * 64 * DH, 64, vtg + (size_t)c * 64, Np, lane);
      load_rows(r0, off[c], off[c + 1] - off[c], 0);
    };
    if constexpr (!PF) {
      BlockFrags<T, DH> fa;
      RowFrags<T, DH> ra;
      for (int a = grab(); a < NZ; a = grab()) {
        load_chunk(fa, ra, nzl[a]);
        process_chunk(fa, ra, nzl[a]);
      }
    } else {
    BlockFrags<T, DH> fa, fb;
    RowFrags<T, DH> ra, rb;
    int a = grab();
    if (a < NZ) load_chunk(fa, ra, nzl[a]);
    while (a < NZ) {
      const int bb = grab();
      if (bb < NZ) load_chunk(fb, rb, nzl[bb]);
      process_chunk(fa, ra, nzl[a]);
      if (bb >= NZ) break;
      a = grab();
      if (a < NZ) load_chunk(fa, ra, nzl[a]);
      process_chunk(fb, rb, nzl[bb]);
    }
    }
  }
  __syncthreads();

  // ------------------------------------------------ write o (8 elements per thread)
  for (int x = tid; x < R * DH / 8; x += 256) {
    const int r = x / (DH / 8), d8 = 8 * (x - r * (DH / 8));
    const int pos = p0 + r / G, hh = r % G;
    float sum[8];
#pragma unroll
    for (int h4 = 0; h4 < 2; ++h4) {
      const int a0 = r * RS + d8 + 4 * h4;
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(accT + a0) +
                       *reinterpret_cast<const f32x4*>(accT + R * RS + a0) +
                       *reinterpret_cast<const f32x4*>(accT + 2 * R * RS + a0) +
                       *reinterpret_cast<const f32x4*>(accT + 3 * R * RS + a0);
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[4 * h4 + j] = s4[j];
    }
    if (pos < N) {
      T* dst = o + (((size_t)b * Hq + g * G + hh) * N + pos) * DH + d8;
      *reinterpret_cast<typename Frag<T>::type*>(dst) = pack8<T>(sum);
    }
  }
}

template <typename T, int G, int DH, int CB>
static size_t fwd_sparse_lds(const Dims& p) {
  constexpr int R = 64 * CB, TP = R / G;
  size_t s = sizeof(float) * (4 * (size_t)R * (DH + 4) + R);
  s += sizeof(int) * (2 * (size_t)p.C + 1);
  s += sizeof(uint16_t) * (size_t)TP * p.K;
  return (s + 15) & ~(size_t)15;
}

// row blocks per wave in the window phase
template <typename T, int DH> struct FwdCB { static constexpr int v = 1; };
template <> struct FwdCB<uint16_t, 64> { static constexpr int v = 2; };

template <typename T, int G, int DH>
static hipError_t fwd_sparse_go(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                         const int32_t* idx, const float* sc, const float* sl, void* o, float* lse,
                         hipStream_t st) {
  constexpr int CB = FwdCB<T, DH>::v;
  constexpr int TP = 64 * CB / G;
  const int ntiles = (p.N + TP - 1) / TP;
  const size_t lds = fwd_sparse_lds<T, G, DH, CB>(p);
  auto kern = k_attn_fwd_sparse<T, G, DH, CB>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(ntiles, p.B * p.Hkv), dim3(256), lds, st, (const T*)q, (const T*)k,
                     (const T*)vt, idx, sc, sl, (T*)o, lse, p.N, Np, p.Hkv, p.K, p.W, p.S, p.scale,
                     ntiles, p.C);
  return hipGetLastError();
}


template <typename T>
static size_t sparse_lds_t(const Dims& p) {
  switch (p.G * 1000 + p.d) {
    case 1064: return fwd_sparse_lds<T, 1, 64, FwdCB<T, 64>::v>(p);
    case 1128: return fwd_sparse_lds<T, 1, 128, FwdCB<T, 128>::v>(p);
    case 2064: return fwd_sparse_lds<T, 2, 64, FwdCB<T, 64>::v>(p);
    case 2128: return fwd_sparse_lds<T, 2, 128, FwdCB<T, 128>::v>(p);
    case 4064: return fwd_sparse_lds<T, 4, 64, FwdCB<T, 64>::v>(p);
    case 4128: return fwd_sparse_lds<T, 4, 128, FwdCB<T, 128>::v>(p);
    default: return (size_t)-1;
  }
}

size_t fwd_sparse_lds_bytes(const Dims& p) {
  return (p.dtype == 1 ? sparse_lds_t<uint16_t>(p) : sparse_lds_t<float>(p)) + 64;
}

template <typename T>
static hipError_t sparse_t(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                           const int32_t* idx, const float* sc, const float* sl, void* o,
                           float* lse, hipStream_t st) {
  switch (p.G * 1000 + p.d) {
    case 1064: return fwd_sparse_go<T, 1, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 1128: return fwd_sparse_go<T, 1, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 2064: return fwd_sparse_go<T, 2, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 2128: return fwd_sparse_go<T, 2, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 4064: return fwd_sparse_go<T, 4, 64>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    case 4128: return fwd_sparse_go<T, 4, 128>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_sparse(const Dims& p, const void* q, const void* k, const void* vt, int Np,
                             const int32_t* idx, const float* sc, const float* sl, void* o,
                             float* lse, hipStream_t st) {
  if (p.dtype == 1) return sparse_t<uint16_t>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
  return sparse_t<float>(p, q, k, vt, Np, idx, sc, sl, o, lse, st);
}

}  // namespace hils
