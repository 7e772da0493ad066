/*
 * hubkv.h -- C ABI of the MI355X (gfx950) KV-cache retention library.
 *
 * The library computes, per KV head, which cached tokens a long-context
 * decoder keeps:
 *   hubkv_score    base scores: attention mass of an observation window
 *   hubkv_refine   HubKV refinement of those scores before Top-K
 *   hubkv_select   per-head Top-K with protected sink and recent tokens
 *   hubkv_refine_select  the two in one call
 *   hubkv_compact  gather of the kept K/V rows into a packed cache
 *   hubkv_score_strided / hubkv_compact_strided
 *                  the same on caller-strided views (token-major, padded)
 *   hubkv_select_layer / hubkv_compact_layer
 *                  a layer's budget shared by its KV heads (per-head floors)
 *   hubkv_nestedkv a second base score from the keys alone (NestedKV)
 *   h2o_step       one streaming (decode) step of H2O greedy eviction
 *   h2o_step_ring  the same step with the recent window kept in a ring of slots
 *   hubkv_score_noalloc
 *                  hubkv_score on a fixed library-held scratch array, for
 *                  callers that cannot allocate
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE memory unless the parameter says "host".
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream) and never synchronises it.
 *   - The library never allocates device memory.  Scratch space is a
 *     caller-provided workspace whose size comes from the matching
 *     *_workspace() query; it must stay alive until the enqueued work has
 *     finished.  The one exception is hubkv_score_noalloc's fixed per-device
 *     scratch array, the library's only mutable global state.
 *   - Host arrays (sequence lengths, kept counts, positions) are read during
 *     the call only.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     validation error nothing is launched, outputs are untouched and a
 *     negative status is returned.  A failed launch returns HUBKV_EHIP and the
 *     HIP error code is kept per thread (hubkv_last_hip_error).  Faults inside
 *     kernels surface at the caller's next synchronisation.
 *   - No C++ exception crosses this interface.
 *
 * Layouts (row-major, the head dimension d contiguous; T = sum of sequence
 * lengths; sequences are packed one after another along the token axis):
 *   Q        [L][Hq][B*W][d]     queries of the last W positions of each sequence
 *   K, V     [L][Hkv][T][d]
 *   s, z     [L][Hkv][T]         fp32
 *   stats    [L][B][Hkv][2]      fp64 {sum_i s_i, sum_i s_i ln s_i}
 *   beta     [L][B][Hkv]         fp32
 *   idx      [L][Hkv][sum_b kept_b]  int32, positions local to their sequence,
 *                                ascending within each sequence
 *   K_out, V_out [L][Hkv][sum_b kept_b][d]
 * Query head h belongs to KV head h / (Hq / Hkv) (contiguous groups).
 * The *_strided calls take the Q, K and V operands as views instead: three
 * element strides (layer, head, row) per operand, a host int64_t[3], d still
 * contiguous.  Element (l, h, r, e) is at base + l*s[0] + h*s[1] + r*s[2] + e,
 * with r the window row b*W + w of Q or the packed token / kept-row index of
 * K and V.  Each stride is a non-negative multiple of 16 bytes; an output
 * view must not map two (layer, head, row) triples onto the same bytes.
 *
 * Limits: 1 <= B <= 64; 1 <= every sequence length < 2^30 (positions and
 * their rounding to tiles are int32 in the kernels; longer sequences return
 * HUBKV_EINVAL); d in {64, 128}; Hq % Hkv == 0; (Hq/Hkv)*W <= 512;
 * W <= every sequence length; element type HUBKV_F32 or HUBKV_BF16; Q/K/V
 * base pointers 16-byte aligned, fp32/int32 arrays 4-byte aligned, fp64
 * arrays 8-byte aligned.
 *
 * Page references are to the public pages this method is described on: the
 * "HubKV walkthrough" page, the "H2O breakdown" page (a walk-through of the
 * heavy-hitter oracle paper) and a general KV-cache survey page.
 */
#ifndef HUBKV_H
#define HUBKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define HUBKV_OK 0
#define HUBKV_EINVAL (-1)     /* a size, count or parameter is out of range      */
#define HUBKV_EDTYPE (-2)     /* unsupported element type or head dimension      */
#define HUBKV_EALIGN (-3)     /* a pointer is null or not aligned as required    */
#define HUBKV_EWORKSPACE (-4) /* workspace missing or smaller than required      */
#define HUBKV_EHIP (-5)       /* a HIP launch failed; see hubkv_last_hip_error() */
#define HUBKV_ESCRATCH (-6)   /* the problem needs more than the fixed scratch   */

/* Element types of Q, K and V. */
#define HUBKV_F32 0
#define HUBKV_BF16 1

/* Workspace bytes hubkv_score needs for this problem (0 on invalid sizes). */
size_t hubkv_score_workspace(int B, const int64_t* seqlens /* host [B] */, int L, int Hq, int Hkv,
                             int W, int d, int dtype);

/*
 * hubkv_score -- base retention score of every cached token.
 *
 * H2O breakdown page, "Observation 2": a token's importance is the attention
 * probability it accumulates over query positions.  KV-cache survey page,
 * section 1.1: the attention is softmax(q K^T / sqrt(d_head)); section 4.3:
 * SnapKV reads this pattern from the prefill queries.  Here the queries are
 * the last W positions of each sequence:
 *   s[l][g][i] = sum over the query heads h of group g and window rows w of
 *                softmax_i( scale * q[l][h][w] . k[l][g][i] ),
 * the softmax over keys i <= N_b - W + w when causal != 0, else over all N_b.
 * head_stats (nullable) receives {sum_i s_i, sum_i s_i ln s_i} per
 * (layer, sequence, KV head); hubkv_refine derives the head weight from it.
 *
 * q, k: element type dtype.  s: fp32 [L][Hkv][T].  workspace: at least
 * hubkv_score_workspace() bytes, 256-byte aligned.
 */
int hubkv_score(const void* q, const void* k, int dtype, int B, const int64_t* seqlens /* host */,
                int L, int Hq, int Hkv, int W, int d, float scale, int causal, float* s,
                double* head_stats /* nullable */, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * hubkv_score_noalloc -- hubkv_score for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, computation and
 * results (bit for bit) as hubkv_score without the workspace: its scratch is
 * a fixed array of HUBKV_SCORE_NOALLOC_BYTES that the library holds on every
 * device it runs on, until the process ends.  The call allocates nothing
 * (no hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks the array's device address up once.  A problem whose
 * hubkv_score_workspace() exceeds that size returns HUBKV_ESCRATCH on the
 * host, before anything is enqueued.  Every call on a device shares that
 * device's array and needs no clearing of it (each call writes every byte it
 * reads), so calls that overlap in time on one device (on different streams,
 * or from several host threads) race on it and must be serialised by the
 * caller.  The device is the one `stream` belongs to (the current device for
 * the null stream).
 */
#define HUBKV_SCORE_NOALLOC_BYTES (16u << 20)

int hubkv_score_noalloc(const void* q, const void* k, int dtype, int B,
                        const int64_t* seqlens /* host */, int L, int Hq, int Hkv, int W, int d,
                        float scale, int causal, float* s, double* head_stats /* nullable */,
                        void* stream);

/*
 * hubkv_score_strided -- hubkv_score on strided Q and K views (same
 * computation, same results bit for bit, same workspace size): a token-major
 * cache [L][T][Hkv][d] is k_strides = {T*Hkv*d, d, Hkv*d}; a cache with
 * room for more tokens per head has a larger head stride.  Strides are
 * host int64_t[3] in elements; invalid strides return HUBKV_EINVAL, strides
 * that are not 16-byte multiples HUBKV_EALIGN.  s and head_stats stay packed.
 */
int hubkv_score_strided(const void* q, const int64_t* q_strides /* host [3] */, const void* k,
                        const int64_t* k_strides /* host [3] */, int dtype, int B,
                        const int64_t* seqlens /* host */, int L, int Hq, int Hkv, int W, int d,
                        float scale, int causal, float* s, double* head_stats /* nullable */,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes hubkv_refine needs (0 on invalid sizes). */
size_t hubkv_refine_workspace(int B, const int64_t* seqlens /* host [B] */, int L, int Hkv);

/*
 * hubkv_refine -- HubKV score refinement before Top-K (HubKV walkthrough,
 * "Method": four steps applied to the base scores, per head):
 *   1 local hubs: token i is a hub when s_i equals the maximum of s over the
 *     window [i - pool/2, i + pool/2] of its own sequence (max-pooling, width
 *     5 on the page; the window is cut at the sequence ends; equal maxima are
 *     all hubs);
 *   2 SMD discount: q_i = s_i for hubs, gamma * s_i otherwise (gamma = 0.5);
 *   3 head calibration: beta_h = clip(sel_h / mean over the layer's KV heads
 *     of sel, beta_lo, beta_hi) with selectivity sel_h = 1 - H(s_h / sum s_h)
 *     / ln N_b (the page asks for a mild, selectivity-based weight clipped to
 *     [0.8, 1.2]); beta_h = 1 when the mean selectivity is not positive;
 *   4 ratio gate: z_i = s_i + r^2 (beta_h q_i - s_i), computed in fp32 as
 *     fma(fl(r*r), fl(beta*q) - s, s).
 * beta comes from beta_in when it is non-null, else from head_stats when it
 * is non-null, else from statistics computed here from s.
 * s, z: fp32 [L][Hkv][T], z must not alias s.  beta_out (nullable) receives
 * the beta used.  pool odd, 1 <= pool <= 63; 0 < gamma <= 1; beta_lo <= beta_hi;
 * 0 <= r <= 1; Hkv <= 1024.
 */
int hubkv_refine(const float* s, int B, const int64_t* seqlens /* host */, int L, int Hkv,
                 const double* head_stats /* nullable */, const float* beta_in /* nullable */,
                 int pool, float gamma, float beta_lo, float beta_hi, float r, float* z,
                 float* beta_out /* nullable */, void* workspace, size_t workspace_bytes,
                 void* stream);

/* Workspace bytes hubkv_select needs (0 on invalid sizes). */
size_t hubkv_select_workspace(int B, const int64_t* seqlens /* host [B] */, int L, int Hkv);

/*
 * hubkv_select -- per-head Top-K with protected windows.
 *
 * HubKV walkthrough: refined scores go to ordinary Top-K pruning, which
 * maximises the modular sum of kept scores.  H2O breakdown page, heavy +
 * recent and per-head sections; KV-cache survey page, sections 4.1-4.2: the
 * first n_sink tokens and the last n_recent tokens of every sequence are
 * always kept.  For each (layer, KV head, sequence b) the kept set is those
 * protected positions plus the kept[b] - |protected| unprotected positions
 * with the largest z, ties to the lower position, NaN lowest, -0 == +0.  The
 * set is written ascending to idx at offset sum_{b' < b} kept[b'].
 * kept: host [B], |protected_b| <= kept[b] <= N_b.  workspace: at least
 * hubkv_select_workspace() bytes, 256-byte aligned (scratch of the call; its
 * content before the call does not matter).  The result is deterministic.
 */
int hubkv_select(const float* z, int B, const int64_t* seqlens /* host */, int L, int Hkv,
                 const int64_t* kept /* host [B] */, int n_sink, int n_recent, int32_t* idx,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes hubkv_refine_select needs (0 on invalid sizes). */
size_t hubkv_refine_select_workspace(int B, const int64_t* seqlens /* host [B] */, int L,
                                     int Hkv);

/*
 * hubkv_refine_select -- hubkv_refine followed by hubkv_select in one call
 * (HubKV walkthrough, "Method": the correction sits between the scorer and an
 * unchanged Top-K).  Arguments as for the two calls; z (required) receives
 * the refined scores and beta_out (nullable) the head weights.  Results
 * equal those of hubkv_refine then hubkv_select bit for bit; the refinement
 * runs inside the selection's first pass.  workspace: at least
 * hubkv_refine_select_workspace() bytes, 256-byte aligned.
 */
int hubkv_refine_select(const float* s, int B, const int64_t* seqlens /* host */, int L, int Hkv,
                        const double* head_stats /* nullable */,
                        const float* beta_in /* nullable */, int pool, float gamma,
                        float beta_lo, float beta_hi, float r, float* z,
                        float* beta_out /* nullable */, const int64_t* kept /* host [B] */,
                        int n_sink, int n_recent, int32_t* idx, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * hubkv_compact -- physically drop evicted tokens (H2O breakdown page, "two
 * code bases": the real-drop variant removes the evicted K/V rows):
 *   K_out[l][g][o_b + j] = K[l][g][cu_b + idx[l][g][o_b + j]], same for V,
 * with cu_b the first token of sequence b and o_b = sum_{b' < b} kept[b'].
 * A bit copy of whole rows; idx as produced by hubkv_select (values must lie
 * in [0, N_b); out-of-range entries are skipped, their rows left untouched).
 */
int hubkv_compact(const void* k_in, const void* v_in, int dtype, const int32_t* idx, int B,
                  const int64_t* seqlens /* host */, const int64_t* kept /* host [B] */, int L,
                  int Hkv, int d, void* k_out, void* v_out, void* stream);

/*
 * hubkv_compact_strided -- hubkv_compact between strided views: the inputs
 * may be token-major or padded caches, and the outputs may be the first
 * sum_b kept_b rows of larger per-head caches (row stride d, head stride the
 * cache capacity times d).  Strides are host int64_t[3] (layer, head, row) in
 * elements.  The output views must not overlap each other or the inputs;
 * only the overlap of distinct rows within one output view is checked.
 */
int hubkv_compact_strided(const void* k_in, const int64_t* k_in_strides /* host [3] */,
                          const void* v_in, const int64_t* v_in_strides /* host [3] */, int dtype,
                          const int32_t* idx, int B, const int64_t* seqlens /* host */,
                          const int64_t* kept /* host [B] */, int L, int Hkv, int d, void* k_out,
                          const int64_t* k_out_strides /* host [3] */, void* v_out,
                          const int64_t* v_out_strides /* host [3] */, void* stream);

/*
 * hubkv_select_layer -- one budget per (layer, sequence), shared by its KV
 * heads.
 *
 * NestedKV summary page, head-wise memory allocation: the layer's budget goes
 * to the (token, head) pairs with the highest scores across the layer, every
 * head keeping a minimum of its own; KV-cache survey page, section 4.4
 * (PyramidKV): the budget is set per layer, here by the caller.  For each
 * (layer l, sequence b), with P_b the protected positions (as hubkv_select)
 * and f_b = min(floor_min, N_b - |P_b|):
 *   every KV head keeps P_b and its f_b best unprotected positions (z
 *   descending, position ascending, NaN lowest, -0 == +0);
 *   the other unprotected (head, position) pairs of the layer compete for
 *   layer_kept[l][b] - Hkv (|P_b| + f_b) places in (z descending, head
 *   ascending, position ascending) order.
 * Each head thus keeps its own top head_kept[l][b][h] positions.
 * z fp32 [L][Hkv][T].  layer_kept host [L][B], row-major, with
 * Hkv (|P_b| + f_b) <= layer_kept[l][b] <= Hkv N_b, L * B <= 256, and the sum
 * over all (l, b) below 2^31.  Outputs: head_kept int32 [L][B][Hkv]; idx
 * int32 [sum of layer_kept]: for each (l, b) in row-major order (offset =
 * sum of the earlier layer_kept), the heads' kept positions head after head,
 * each head's ascending.  workspace >= hubkv_select_layer_workspace(), 256-B
 * aligned; it holds the search state and is fully rewritten by every call.
 * Deterministic.
 */
size_t hubkv_select_layer_workspace(int B, const int64_t* seqlens /* host */, int L, int Hkv);

int hubkv_select_layer(const float* z, int B, const int64_t* seqlens /* host */, int L, int Hkv,
                       const int64_t* layer_kept /* host [L][B] */, int n_sink, int n_recent,
                       int floor_min, int32_t* idx, int32_t* head_kept, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * hubkv_compact_layer -- the K/V rows of a hubkv_select_layer result, packed
 * in idx's order: row o of (l, b, h) is K[l][h][cu_b + idx[o]] (same for V),
 * k_out/v_out [sum of layer_kept][d].  head_kept (device) says which head
 * each row belongs to; layer_kept (host) must be the one given to
 * hubkv_select_layer.  Positions outside [0, N_b) are skipped.
 */
int hubkv_compact_layer(const void* k_in, const void* v_in, int dtype, const int32_t* idx,
                        const int32_t* head_kept, int B, const int64_t* seqlens /* host */, int L,
                        int Hkv, const int64_t* layer_kept /* host [L][B] */, int d, void* k_out,
                        void* v_out, void* stream);

/*
 * hubkv_nestedkv -- key-only base score (NestedKV summary page: continuum
 * memory state, adaptive blending and surprise-gated routing).  Per (layer l,
 * KV head g, sequence b), with k^_i = k_i / |k_i| (0 for a zero key):
 *   mu_s = mean of k^ over the sequence (stable memory);
 *   mu_e(i) = mean of k^ over i's block, blocks of ceil(N_b / nblocks) keys
 *             from the start (episodic memory);
 *   mu_c(i) = mean of k^ over the `window` keys ending at i (current memory);
 *   a_x(i) = -cos(k^_i, mu_x), 0 when either vector is zero;
 *   w = softmax over x of (max_i a_x - min_i a_x + log_prior[x]);
 *   s_i = max(a_s, a_e, a_c) when the population standard deviation of the
 *         three exceeds theta, else sum_x w_x a_x.
 * The pages give neither the prior nor the threshold: both are arguments
 * (log_prior host [3], nullable = zeros).  k [L][Hkv][T][d] (dtype); s fp32
 * [L][Hkv][T]; anomalies (nullable) fp32 [L][Hkv][T][3] (a_s, a_e, a_c);
 * weights (nullable) fp32 [L][B][Hkv][3].  window must be 64; 1 <= nblocks
 * <= 4096.  The scores can go to hubkv_select / hubkv_select_layer as they
 * are (any real values order); hubkv_refine expects non-negative scores.
 * workspace >= hubkv_nestedkv_workspace(), 256-B aligned.  Deterministic.
 */
size_t hubkv_nestedkv_workspace(int B, const int64_t* seqlens /* host */, int L, int Hkv, int d,
                                int nblocks);

int hubkv_nestedkv(const void* k, int dtype, int B, const int64_t* seqlens /* host */, int L,
                   int Hkv, int d, int nblocks, int window,
                   const float* log_prior /* host [3], nullable */, float theta, float* s,
                   float* anomalies /* nullable */, float* weights /* nullable */,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * h2o_step -- one decode step of H2O greedy eviction on a fixed-slot cache.
 *
 * H2O breakdown page, "greedy eviction" (Algorithm 1 description), the heavy
 * + recent section and the FlexGen section (preallocated slots; the evicted
 * token's slot is overwritten by the new token; accumulated scores ride on
 * the attention computation).  Independently per (sequence b, KV head g):
 *   p_h   = softmax over the occupied slots (and the new token itself when
 *           include_self != 0) of scale * q[b][h] . k_cache[b][g][slot], for
 *           the query heads h of the group;
 *   acc  += sum_h p_h on the occupied slots;
 *   the new token t[b] enters with acc = include_self ? sum_h p_h(new) : 0;
 *   if a slot is empty (pos < 0) the lowest such slot takes it; otherwise the
 *   token with the smallest acc among positions in [n_sink, t - n_recent]
 *   (the new token included when it qualifies) is evicted, ties to the
 *   oldest position, and its slot takes the new token (K/V row, acc, pos).
 * q [B][Hq][d], k_new/v_new [B][Hkv][d] (dtype); k_cache/v_cache
 * [B][Hkv][C][d] (dtype), acc fp32 and pos int32 [B][Hkv][C] (-1 = empty),
 * all updated in place.  t: host [B] positions of the new tokens.
 * evicted (nullable) [B][Hkv]: evicted position or -1.  probs (nullable)
 * [B][Hq][C+1] fp32: this step's probabilities per slot (0 for empty slots)
 * and, last, the new token's own probability.
 * out (nullable) [B][Hq][d] fp32: the step's attention output -- the decode
 * attention of the KV-cache page (section 1.1) over the retained tokens only
 * (H2O breakdown page, problem statement: evicted tokens leave the
 * normaliser): out[b][h] = sum over occupied slots of p_h(slot) *
 * v_cache[b][g][slot], plus p_h(new) * v_new[b][g] when include_self, with
 * the same p_h that are added to acc, on the cache before the new token is
 * written.  All zeros when there is nothing to attend to.
 * Requires C >= n_sink + n_recent, Hq/Hkv <= 16 and (Hq/Hkv + 1) * C <= 16384
 * (the logits and the slot positions of one (sequence, KV head) sit in LDS).
 * Buffers must not overlap (out, probs and evicted are written while the
 * caches are read).
 */
int h2o_step(const void* q, const void* k_new, const void* v_new, int dtype, void* k_cache,
             void* v_cache, float* acc, int32_t* pos, const int64_t* t /* host [B] */, int B,
             int Hq, int Hkv, int d, int C, int n_sink, int n_recent, float scale,
             int include_self, int32_t* evicted /* nullable */, float* probs /* nullable */,
             float* out /* nullable */, void* stream);

/*
 * h2o_step_ring -- h2o_step on the ring slot layout of the H2O breakdown
 * page's FlexGen section (the recent region is a circular queue of slots
 * whose head and tail advance in O(1)).  Slots [0, C - n_recent) hold heavy
 * tokens; slots [C - n_recent, C) are the ring, and position p sits in ring
 * slot C - n_recent + p mod n_recent.  The new token t[b] takes the ring slot
 * of position t[b] - n_recent, the token that leaves the recent window; that
 * token moves (K/V row, acc, pos copied) to the lowest free heavy slot, or,
 * with the heavy slots full, the token with the smallest acc among the heavy
 * positions in [n_sink, t - n_recent] and the leaving token itself is
 * evicted (ties to the oldest position); when the victim is a heavy token,
 * the leaving token takes its slot.  The candidates are the fixed layout's,
 * so a cache driven by this call from empty, with t advancing by one per
 * step, retains the same tokens with the same acc as h2o_step (in other
 * slots; probs follow this layout's slots).  Arguments, outputs and limits
 * as for h2o_step, plus 1 <= n_recent < C.  A cache must be driven by one
 * layout from empty.
 */
int h2o_step_ring(const void* q, const void* k_new, const void* v_new, int dtype, void* k_cache,
                  void* v_cache, float* acc, int32_t* pos, const int64_t* t /* host [B] */, int B,
                  int Hq, int Hkv, int d, int C, int n_sink, int n_recent, float scale,
                  int include_self, int32_t* evicted /* nullable */, float* probs /* nullable */,
                  float* out /* nullable */, void* stream);

/* Number of protected positions of a sequence of length N (host helper). */
int64_t hubkv_protected_count(int64_t N, int n_sink, int n_recent);

/* Static text for a status code. */
const char* hubkv_strerror(int status);

/* hipError_t behind the calling thread's last HUBKV_EHIP (0 if none). */
int hubkv_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int hubkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HUBKV_H */
