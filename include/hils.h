/*
 * hils.h - C ABI of the HiLS (Hierarchical Landmark Sparse) attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is that of "Hierarchical Sparse Attention Done Right: Toward
 * Infinite Context Modeling" (Hu et al.). Each query, offset by a low-rank
 * calibration (Q-Cal), scores every distant chunk with a surrogate built from
 * the chunk's landmark key and entropy bias, keeps the top-K chunks, runs exact
 * softmax attention inside each of them and inside a local sliding window, and
 * fuses the per-chunk outputs with a softmax over the chunk scores and the
 * window's log-sum-exp.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; every tensor
 *   is dense row-major with the layout given below. The library allocates no
 *   device memory and keeps no state between calls: scratch comes from the
 *   caller's workspace, sized by hils_workspace_size() for the same problem
 *   and op. The workspace must be 256-byte aligned.
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *   and the call returns without synchronising. Calls on different streams
 *   with different workspaces may run concurrently: everything a call uses
 *   comes through its arguments (the library holds no mutable state).
 * - Validation happens before anything is enqueued and has no side effects.
 *   Errors: HILS_ERR_INVALID (null required pointer, size <= 0, Hq % Hkv != 0,
 *   Nq/Nk inconsistent with the op), HILS_ERR_UNSUPPORTED (a valid problem
 *   outside what the kernels implement, e.g. d not in {64,128}, S != 64,
 *   K > 64, Hq/Hkv not in {1,2,4,8}; hils_attn_fwd and hils_attn_bwd accept
 *   exactly the same problems), HILS_ERR_WORKSPACE (ws too small or
 *   misaligned), HILS_ERR_HIP (a kernel launch failed). A fault inside a
 *   kernel surfaces at the caller's next synchronisation. Nothing prints,
 *   aborts or throws across this boundary.
 * - A sequence shorter than one chunk (Nk < S) has no complete chunk: the
 *   chunk tensors (kL, e, their gradients, landmark queries) are then empty
 *   and may be NULL.
 *
 * Notation (the paper's): B batch, Hq query heads, Hkv KV heads, G = Hq/Hkv
 * (query head h uses KV head h / G), d head dim, S chunk size, C = Nk / S
 * complete chunks, K top-K, W window, D hidden size, r Q-Cal rank,
 * scale = 1/sqrt(d) unless given.
 *
 * Geometry (a reading of the paper's chunk/window statement, where the pages
 * leave the boundary open): the query at position i sees the distant chunks
 * c < n_dist(i) = max(0, floor((i - W + 1) / S)) (chunks whose newest token is
 * at least W positions older than i) and the window of tokens
 * [n_dist(i) * S, i].
 *
 * Layouts
 *   q        [B, Hq, Nq, d]      (decode: [B, Hq, d])
 *   k, v     [B, Hkv, Nk, d]
 *   kL       [B, Hkv, C, d]      landmark key of each complete chunk
 *   e        [B, Hkv, C]         entropy bias of each complete chunk
 *   h        [B, Nq, D]          hidden state feeding Q-Cal (decode: [B, D])
 *   W_down   [Hq, r, D]          (qcal_shared: [r, D])
 *   W_up     [Hq, d, r]          (qcal_shared: [d, r])
 *   o        [B, Hq, Nq, d]      in the input dtype (decode: [B, Hq, d])
 *   lse      [B, Hq, Nq] fp32    fusion log-normaliser L
 *   topk_idx [B, Hkv, Nq, K] int32, ascending chunk ids, -1 in unused slots
 *   gradients: fp32, same shapes as the tensors they belong to.
 */
#ifndef HILS_H_
#define HILS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HILS_OK = 0,
  HILS_ERR_INVALID = 1,
  HILS_ERR_UNSUPPORTED = 2,
  HILS_ERR_WORKSPACE = 3,
  HILS_ERR_HIP = 4
} hils_status;

typedef enum { HILS_FP32 = 0, HILS_BF16 = 1 } hils_dtype;

/* Operation ids for hils_workspace_size. */
typedef enum { HILS_OP_ROUTE = 0, HILS_OP_FWD = 1, HILS_OP_BWD = 2, HILS_OP_DECODE = 3 } hils_op;

/*
 * Measurement hook (not part of the method), per call: ids of the launch
 * steps whose device time a caller can bracket with its own events.
 */
typedef enum {
  HILS_STEP_QCAL = 0,         /* Q-Cal (fp32 calibrated queries, or u) */
  HILS_STEP_ROUTE = 1,        /* scoring + GQA max + top-K (prefill) */
  HILS_STEP_ATTN_FWD = 2,     /* every attention launch of a prefill forward */
  HILS_STEP_DECODE = 3,       /* the whole decode step after Q-Cal */
  HILS_STEP_BWD = 4,          /* the whole backward */
  HILS_STEP_LANDMARK_FWD = 5, /* landmark summary */
  HILS_STEP_LANDMARK_BWD = 6, /* its backward */
  HILS_STEP_HOPE = 7,         /* HoPE rotation */
  HILS_STEP_WINDOW = 8,       /* prefill forward: the one launch that ends in the
                                 fusion (chunk-major: window + fusion; the
                                 query-major strategies: window + selected
                                 chunks + fusion) */
  HILS_STEP_CHUNKS = 9,       /* chunk-major forward: the selected-chunk launch */
  HILS_STEP_PREP = 10,        /* prefill forward: the V^T copy, and for
                                 chunk-major the inverse index and work items */
  HILS_STEP_COUNT = 11
} hils_step;

/*
 * Caller-owned events (hipEvent_t handles, NULL = not timed) for one call:
 * a call records start[s] on its stream right before the launches of step s
 * and stop[s] right after them. The library keeps no pointer past the call.
 */
typedef struct {
  void* start[HILS_STEP_COUNT];
  void* stop[HILS_STEP_COUNT];
} hils_timing;

/*
 * Forward strategy (how the prefill forward is scheduled, not what it
 * computes; every strategy gives the same per-query result):
 *   HILS_FWD_AUTO (0)        chosen by shape;
 *   HILS_FWD_UNION (1)       packed union (the paper's Fig. 4 kernel design):
 *                            a tile of adjacent queries streams the union of
 *                            their selected chunks through LDS once;
 *   HILS_FWD_COMPACT (2)     per query tile, each selected chunk's rows are
 *                            packed into dense row blocks;
 *   HILS_FWD_CHUNK_MAJOR (3) chunk-major: every selected chunk is loaded once
 *                            and serves all the rows that selected it; the
 *                            per-chunk outputs are fused with the window's in
 *                            a second pass (for long sequences, where adjacent
 *                            queries share few chunks).
 */
typedef enum {
  HILS_FWD_AUTO = 0,
  HILS_FWD_UNION = 1,
  HILS_FWD_COMPACT = 2,
  HILS_FWD_CHUNK_MAJOR = 3
} hils_fwd_strategy;

typedef struct {
  int32_t dtype;        /* hils_dtype of q, k, v, kL, e, h, W_down, W_up, o, dO */
  int32_t B, Hq, Hkv, d;
  int32_t Nq, Nk;       /* prefill/backward: Nq == Nk (query i at position i);
                           decode: Nq == 1, Nk = cache capacity */
  int32_t S, K, W;      /* chunk size, top-K (>= 1), window in tokens (>= 1) */
  int32_t D, r;         /* Q-Cal hidden size and rank; r == 0 => no Q-Cal */
  int32_t qcal_shared;  /* 1 => one (W_down, W_up) pair shared by all heads:
                           W_down [r, D], W_up [d, r], dW_down / dW_up the same
                           shapes (the sum of the heads' gradients); 0 or 1 */
  float scale;          /* 0 => 1/sqrt(d) */
  int32_t fwd_strategy; /* hils_fwd_strategy of the prefill forward (0 = auto);
                           hils_workspace_size(HILS_OP_FWD) sizes for it */
  const hils_timing* timing; /* NULL, or events to record around this call's steps */
} hils_problem;

/* Text for a status code (static storage). */
const char* hils_status_string(hils_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t hils_version(void);

/* Bytes of workspace that `op` needs for problem `p` (written to *bytes). */
hils_status hils_workspace_size(const hils_problem* p, int32_t op, size_t* bytes);

/*
 * The forward strategy hils_attn_fwd runs for problem `p` (p->fwd_strategy,
 * or the one HILS_FWD_AUTO resolves to by shape), written to *strategy as a
 * hils_fwd_strategy other than AUTO. Errors as hils_workspace_size for
 * HILS_OP_FWD: HILS_ERR_INVALID for a null or malformed problem,
 * HILS_ERR_UNSUPPORTED when no strategy runs it.
 */
hils_status hils_fwd_strategy_of(const hils_problem* p, int32_t* strategy);

/*
 * Routing only: Q-Cal, surrogate scores, GQA max and top-K selection
 * (paper: Q-Cal worked example and surrogate-score step of "The
 * HiLS-Attention Mechanism"; Fig. 3; GQA paragraph of the Q-Cal section).
 *   s_{h,c} = scale * q_hat_h . kL_{g(h),c} + e_{g(h),c}, c < n_dist(i),
 *   q_hat = q + W_up (W_down h) (q_hat = q when r == 0);
 *   the group's selection score is the max over its heads; the K best
 *   (score desc, lower index first on ties) distant chunks are kept.
 * Outputs: topk_idx (required); topk_score [B, Hq, Nq, K] fp32 (nullable):
 * s_{h,c} of each selected chunk in topk_idx order (NaN in unused slots).
 */
hils_status hils_route(const hils_problem* p, const void* q, const void* kL, const void* e,
                       const void* h, const void* W_down, const void* W_up, int32_t* topk_idx,
                       float* topk_score, void* ws, size_t ws_bytes, void* stream);

/*
 * Prefill forward (paper Fig. 3 and the engineersofai abstract: per-chunk
 * attention fused by the retrieval scores). For each row (b, h, i):
 *   L = log( sum_{c in T} exp(s_{h,c}) + exp(lse_W) ),
 *   o = sum_{c in T} exp(s_{h,c} - L) O_c + exp(lse_W - L) O_W,
 * with O_c, lse_c the exact softmax attention of the raw q over chunk c's
 * S tokens and O_W, lse_W over the window. Writes o, lse and topk_idx (all
 * required); topk_idx and lse are the saved tensors hils_attn_bwd consumes.
 * topk_idx (here, in hils_route and hils_attn_bwd) needs only int32
 * alignment: the kernels move the ids as 16-byte vectors where the pointer
 * is 16-byte aligned and K is a multiple of 4, one at a time otherwise.
 */
hils_status hils_attn_fwd(const hils_problem* p, const void* q, const void* k, const void* v,
                          const void* kL, const void* e, const void* h, const void* W_down,
                          const void* W_up, void* o, float* lse, int32_t* topk_idx, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Training backward of hils_attn_fwd with the selection topk_idx held fixed
 * (the paper trains the landmark keys end to end through the fusion softmax,
 * Fig. 3 caption; top-K itself is not differentiated). Inputs are the forward
 * inputs, its lse and topk_idx, and the upstream gradient dO [B, Hq, Nq, d].
 * o may be NULL and is not read: dO . o is recomputed in fp32 from the
 * attention weights, so the rounding of o does not enter the gradients.
 * Outputs (fp32, overwritten, all required except dh): dq, dk, dv, dkL, de;
 * dW_down, dW_up when r > 0 (ignored when r == 0); dh [B, Nq, D] (nullable).
 */
hils_status hils_attn_bwd(const hils_problem* p, const void* q, const void* k, const void* v,
                          const void* kL, const void* e, const void* h, const void* W_down,
                          const void* W_up, const void* o, const float* lse,
                          const int32_t* topk_idx, const void* dO, float* dq, float* dk, float* dv,
                          float* dkL, float* de, float* dW_down, float* dW_up, float* dh,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Decode step: one new query per sequence at position seq_len[b]-1, its key
 * and value already in the cache (the paper's per-token decode, Fig. 6).
 * q [B, Hq, d]; k_cache, v_cache [B, Hkv, Nk, d]; seq_len [B] int32 device
 * (NULL => every sequence holds Nk tokens; each must be in [1, Nk]);
 * kL [B, Hkv, Nk/S, d], e [B, Hkv, Nk/S] (only the first seq_len/S are read);
 * h [B, D] (only when r > 0). Writes o [B, Hq, d], lse [B, Hq] and, if
 * non-NULL, topk_idx [B, Hkv, K].
 */
hils_status hils_decode(const hils_problem* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* seq_len, const void* kL, const void* e,
                        const void* h, const void* W_down, const void* W_up, void* o, float* lse,
                        int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * hils_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and outputs as hils_decode, with the workspace
 * replaced by a static device buffer of HILS_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its address is
 * looked up once per device, on the first call with that device current; the
 * calling thread's current device must be the stream's). The call itself
 * allocates nothing. Every call on one GPU shares that GPU's buffer: calls
 * that overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller; a call may start once the previous one's work is
 * ordered before it on the stream. Errors: those of hils_decode, plus
 * HILS_ERR_WORKSPACE when hils_workspace_size(p, HILS_OP_DECODE) exceeds
 * HILS_NOALLOC_SCRATCH_BYTES (e.g. 32 sequences x 32 heads x d = 128 at
 * K = 32 and a 1024-token window need ~31 MB and fit), and HILS_ERR_HIP when
 * the buffer's address cannot be obtained.
 */
#define HILS_NOALLOC_SCRATCH_BYTES (64u << 20)
hils_status hils_decode_noalloc(const hils_problem* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* seq_len, const void* kL,
                                const void* e, const void* h, const void* W_down, const void* W_up,
                                void* o, float* lse, int32_t* topk_idx, void* stream);

/*
 * Decode step over a paged KV cache (the serving layout of the pages'
 * released backend, whose page size equals the 64-token chunk: one chunk is
 * one page). Same method and outputs as hils_decode; only where the cache
 * rows live differs:
 *   k_pages, v_pages [P, Hkv, S, d]   tokens of page p
 *   kL_pages [P, Hkv, d], e_pages [P, Hkv]   landmark key and bias of page p
 *   page_table [B, max_pages] int32    page of chunk c of sequence b (tokens
 *                                      c*S .. c*S+S-1); entries for chunks at
 *                                      or past ceil(seq_len[b] / S) are not read
 *   seq_len [B] int32 (required), each in [1, max_pages * S].
 * p->Nk must equal max_pages * S (the per-sequence capacity; it sizes the
 * workspace like hils_decode's). Page ids must lie in [0, P) (not checked).
 * kL_pages / e_pages are read only for complete chunks below the distant
 * boundary. Errors as hils_decode, plus HILS_ERR_INVALID for a null
 * page_table or seq_len or an inconsistent max_pages.
 */
hils_status hils_decode_paged(const hils_problem* p, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_len, const void* kL_pages, const void* e_pages,
                              const void* h, const void* W_down, const void* W_up, void* o,
                              float* lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * Landmark summary (paper: "The HiLS-Attention Mechanism", the landmark
 * worked example; the overview's first-order Taylor expansion of a chunk's
 * attention mass around its landmark query). For every complete chunk c of
 * every (b, KV head), with the chunk's S tokens t:
 *   s_t = scale * qL_c . k_t,  p = softmax(s),
 *   kL_c = sum_t p_t k_t,      e_c = -sum_t p_t log p_t   (fp32 arithmetic).
 * qL [B, Hkv, C, d] holds one landmark query per chunk and KV head; k
 * [B, Hkv, Nk, d]; C = Nk / S. Outputs kL [B, Hkv, C, d] and e [B, Hkv, C]
 * in the problem dtype (rounded to nearest even from fp32: the layout and
 * dtype hils_route, hils_attn_fwd and hils_decode take), and, when non-NULL,
 * the same values in fp32 (kL32, e32). Only dtype, B, Hkv, d, Nk, S and scale
 * of the problem are read (Hq, Nq, K, W, D, r are ignored); no workspace.
 * qL, k, kL and kL32 must be 16-byte aligned (rows move as 16-byte vectors).
 * Errors: HILS_ERR_INVALID (null qL, k, kL or e; B, Hkv, d or Nk <= 0; bad
 * scale; a misaligned pointer), HILS_ERR_UNSUPPORTED (d not in {64, 128},
 * S != 64).
 */
hils_status hils_landmark_fwd(const hils_problem* p, const void* qL, const void* k, void* kL,
                              void* e, float* kL32, float* e32, void* stream);

/*
 * Backward of hils_landmark_fwd (the chain rule; the pages print none): from
 * dkL [B, Hkv, C, d] and de [B, Hkv, C] (fp32, as hils_attn_bwd writes them),
 * with s, p of the forward recomputed in fp32 and sbar = sum_t p_t s_t:
 *   ds_t  = p_t (dkL_c . k_t - dkL_c . kL_c - de_c (s_t - sbar)),
 *   dqL_c = scale sum_t ds_t k_t                       (written, fp32),
 *   dk_t += scale ds_t qL_c + p_t dkL_c                (ADDED into dk, fp32
 *           [B, Hkv, Nk, d], e.g. after hils_attn_bwd wrote it; tokens past
 *           C * S are not touched).
 * Same problem fields and errors as hils_landmark_fwd (null dkL, de, dqL or
 * dk, or a misaligned qL, k, dkL, dqL or dk, is HILS_ERR_INVALID).
 */
hils_status hils_landmark_bwd(const hils_problem* p, const void* qL, const void* k,
                              const float* dkL, const float* de, float* dqL, float* dk,
                              void* stream);

/*
 * HoPE, the partial rotary position encoding of queries and keys (paper:
 * "Implementation and Training Recipes", HoPE; dev.to summary, "Engineering
 * Details", Hierarchical Positional Encoding): the rotary frequencies
 * theta_j = base^(-2j/d), j < d/2, are kept only where the period
 * 2 pi / theta_j fits the training length; the other pairs carry no position
 * (NoPE). For row (b, h, n) of x [B, H, N, d] at position p = pos[b, n]
 * (pos == NULL: p = n) and each rotating pair (a, b):
 *   y_a = x_a cos(p theta_j) - x_b sin(p theta_j)
 *   y_b = x_a sin(p theta_j) + x_b cos(p theta_j)
 * (angle -p theta_j when inverse = 1: the transpose, which maps gradients of
 * y to gradients of x); NoPE pairs are copied. Pairs are (j, j + d/2), or
 * (2j, 2j + 1) when interleaved = 1. The angle is reduced to a fraction of a
 * turn in fp64, the rotation is computed in fp32 and rounded to the dtype.
 * Apply it to q and k before Q-Cal, routing, the landmark summary and the
 * attention calls (and its inverse to dq and dk after the backward); decode
 * rotates the new query at position seq_len - 1.
 * y may be x (in place); x and y must be 16-byte aligned, pos (int32 [B, N])
 * holds positions >= 0. B, H or N == 0: nothing to do (x and y may be NULL).
 * Errors: HILS_ERR_INVALID (null p; null x or y with work to do; negative sizes; base not finite
 * or <= 1; train_len < 0; flags not 0 / 1; misaligned x or y; more than
 * 2^31 16-byte units), HILS_ERR_UNSUPPORTED (d not in {64, 128}).
 */
typedef struct {
  int32_t dtype;       /* hils_dtype of x and y */
  int32_t B, H, N, d;
  float base;          /* rotary base, e.g. 10000 */
  int32_t train_len;   /* training context length (tokens) */
  int32_t interleaved; /* 0: pairs (j, j + d/2); 1: pairs (2j, 2j + 1) */
  int32_t inverse;     /* 1: rotate by -angle (gradients) */
  const hils_timing* timing; /* NULL, or events around the rotation (HILS_STEP_HOPE) */
} hils_hope_params;
hils_status hils_hope(const hils_hope_params* p, const void* x, void* y, const int32_t* pos,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HILS_H_ */
