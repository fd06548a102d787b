/*
 * retopk.h - C ABI of the ReTopK decode-step attention library (MI355X, gfx950).
 *
 * The method is the one of "Recall Before You Rank: Similarity-Guided Top-K
 * Reuse for Efficient Long-Context Attention" (ReTopK). For each query head a
 * decode step:
 *   1. normalises the current query and compares it by cosine similarity with a
 *      bounded FIFO cache of C normalised past queries (Methodology, Eqs. 5-6);
 *   2. takes the R most similar cache entries and rho_max (Eq. 7);
 *   3. unions their stored supports with the W most recent token positions and
 *      de-duplicates the result into the candidate set A_t (Eqs. 8-9);
 *   4. scores the current query exactly against the candidate keys only (Eq. 10);
 *   5. reranks to exactly K indices (Eq. 11);
 *   6. computes softmax-weighted values over that support (Eq. 12);
 * and takes the exact path - full-history scores (Eq. 4) and global Top-K
 * (Eq. 1) - when rho_max < tau or on every T_r-th decode step (Reliable Reuse
 * via Fallback and Refresh, Eq. 13). The cache is updated after either path.
 * The path is decided on the device; a step performs no host synchronisation
 * and no allocation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types. bf16 tensors are passed as uint16_t bit patterns. All tensors are
 *   dense, row-major, C-contiguous, in device memory unless stated otherwise.
 * Shapes. B = batch, Hq = query heads, Hkv = KV heads (Hq % Hkv == 0, Hq/Hkv
 *   <= 16), D = head dimension (must be 128), Lmax = max_len.
 *     q      [B, Hq, D]          bf16, post-positional-encoding query
 *     k, v   [B, Hkv, Lmax, D]   bf16 KV cache; query head h reads KV head
 *                                 h / (Hq / Hkv) (contiguous GQA groups)
 *     out    [B, Hq, D]          float32 attention output
 *   q, k and v must be 16-byte aligned; out 4-byte aligned.
 * Positions. Token indices are 0-based. A call with visible length L reads
 *   key/value rows 0 .. L-1 only; the caller has already written the current
 *   token's key and value at row L-1, so the query attends to itself. The
 *   recent window is rows max(0, L-W) .. L-1. L must not decrease between
 *   calls on one handle.
 * Ties. Top-K ties go to the lower token index; TopR ties go to the older
 *   cache entry. Supports are stored and returned in ascending index order.
 *   When fewer than K keys (or candidates) exist, all of them are taken.
 * Ownership. The caller owns q, k, v, out and every host buffer. The library
 *   owns the handle and all device state below it (cache and workspaces,
 *   allocated once by retopk_create and freed by retopk_destroy).
 * Streams. `stream` is a hipStream_t passed as void*; NULL means the default
 *   stream. Work is enqueued asynchronously; errors of the asynchronous work
 *   itself appear at the next synchronising call. A handle must be used from
 *   one host thread and one stream at a time; calls that overlap on one
 *   handle race.
 * Co-residency. retopk_decode_step, retopk_exact_topk_attn and
 *   retopk_init_from_prefill are each one kernel launch whose work groups hand
 *   results to one another through device memory: the work groups of an
 *   exact KV group wait for each other's scores and survivors. The grid is
 *   sized so that all of them fit on the device at once (at most one
 *   work group per compute unit besides the head work groups, which never
 *   wait), which holds when nothing else runs on the GPU during the call.
 *   Work on other streams or from other processes that holds compute units
 *   meanwhile can keep some work groups from starting; every wait is bounded
 *   (about 200 ms), so the call still ends, but then its exact heads are not
 *   finished, their outputs and cache entries are not valid and the sticky
 *   device error word is set (retopk_read_device_error). Callers that must
 *   share the GPU check that word after the steps they need to trust.
 * Errors. Every entry point returns a retopk_status. Arguments are checked
 *   before any device work is enqueued; on error nothing is enqueued and the
 *   handle's state is unchanged. retopk_last_error() gives a message for the
 *   calling thread's last failure. No C++ exception crosses the ABI.
 */
#ifndef RETOPK_H
#define RETOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum retopk_status {
  RETOPK_OK = 0,
  RETOPK_INVALID_ARG = 1,      /* null or misaligned pointer, inconsistent parameters */
  RETOPK_OUT_OF_RANGE = 2,     /* a length, step or index outside its valid range   */
  RETOPK_HIP_ERROR = 3,        /* a HIP runtime call or kernel launch failed         */
  RETOPK_NOT_INITIALIZED = 4,  /* null handle                                        */
  RETOPK_NO_DEVICE = 5         /* no usable GPU                                      */
} retopk_status;

/* Method and shape parameters (defaults of the paper's experiments:
 * K = 512, C = W = 32, R = 4, tau = 0.85, T_r = 128). */
typedef struct retopk_params {
  int32_t batch;          /* B >= 1                                              */
  int32_t n_q_heads;      /* Hq >= 1                                             */
  int32_t n_kv_heads;     /* Hkv >= 1, divides Hq, Hq / Hkv <= 16, B*Hkv <= 1024 */
  int32_t head_dim;       /* D, must be 128                                      */
  int32_t max_len;        /* Lmax: rows of the k / v buffers, 1 .. 2^24          */
  int32_t top_k;          /* K, 1 .. 8192                                        */
  int32_t cache_cap;      /* C, 1 .. 64 (query-support cache capacity, Eq. 5)    */
  int32_t window;         /* W >= 0 (recent-token window, Eq. 8)                 */
  int32_t top_r;          /* R, 1 .. C (retrieved entries, Eq. 7)                */
  int32_t refresh_every;  /* T_r >= 0; 0 disables scheduled refresh (Eq. 13)     */
  double  tau;            /* similarity threshold: rho_max < tau takes the exact
                             path (Eq. 13); compared against rho in float64      */
  int32_t retrieval;      /* RETOPK_RETRIEVE_SIMILAR (0, the method): R_t = the R
                             entries most similar to q_t (Eq. 7), rho_max over
                             all entries; RETOPK_RETRIEVE_RECENT (1, the component
                             ablation of the Experiments' Table 3): R_t = the R
                             newest entries, newest first, and rho_max over them
                             only                                                */
} retopk_params;

enum { RETOPK_RETRIEVE_SIMILAR = 0, RETOPK_RETRIEVE_RECENT = 1 };

typedef struct retopk_handle retopk_handle;

/* Stable message for a status code. */
const char* retopk_status_string(retopk_status s);

/* Message of the calling thread's last failed call ("" if none). */
const char* retopk_last_error(void);

/* Create a handle on the current HIP device: validates *params and allocates
 * the per-head query-support caches (empty) and every workspace at worst-case
 * size (R*K + W candidates, Lmax scores per head), plus one pinned,
 * device-mapped host word through which decode steps report their exact KV
 * groups to size later launches. Synchronous. On success *out receives the
 * handle; on failure *out is set to NULL. */
retopk_status retopk_create(const retopk_params* params, retopk_handle** out);

/* Free the handle and all its device memory (synchronises the device first).
 * A NULL handle is ignored. */
void retopk_destroy(retopk_handle* h);

/* Initialise every cache from the final n0 = min(C, prompt_len) prompt queries
 * ("initialized from the final C prompt tokens during prefill", Query-support
 * cache paragraph). q_tail is bf16 [B, Hq, n0, D], holding the queries of
 * prompt positions prompt_len - n0 .. prompt_len - 1 in order. The entry of
 * position p is (q_p / ||q_p||, causal Exact Top-K support of q_p over keys
 * 0 .. p). Entries are pushed oldest first, replacing any previous contents.
 * 1 <= prompt_len <= Lmax. Asynchronous on `stream`. */
retopk_status retopk_init_from_prefill(retopk_handle* h, const uint16_t* q_tail,
                                       const uint16_t* k, int32_t prompt_len, void* stream);

/* One ReTopK decode step (Eqs. 5-13) for all B * Hq heads at visible length
 * `length` (1 .. Lmax) and decode-step offset t_dec (>= 1; refresh fires when
 * T_r > 0 and t_dec is a multiple of T_r). Writes out [B, Hq, D] and pushes
 * (q_bar_t, S_hat_t) into every head's cache. The path decision stays on the
 * device: no host synchronisation, no allocation. Asynchronous on `stream`.
 * When the handle records statistics, step t_dec is stored in slot
 * (t_dec - 1) mod 4096 of the statistics ring. */
retopk_status retopk_decode_step(retopk_handle* h, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, int32_t length, int32_t t_dec,
                                 float* out, void* stream);

/* Exact Top-K attention baseline (Problem Setup: Eq. 4 scores over all
 * `length` keys, Eq. 1 global Top-K, then Eq. 12): the same full-history
 * kernels the exact path of retopk_decode_step uses, with every head exact and
 * the cache left untouched. out [B, Hq, D] float32. sel_out, if not NULL,
 * receives the selected indices, int32 [B, Hq, K] ascending; rows with fewer
 * than K keys are padded with -1. Asynchronous on `stream`. */
retopk_status retopk_exact_topk_attn(retopk_handle* h, const uint16_t* q, const uint16_t* k,
                                     const uint16_t* v, int32_t length, float* out,
                                     int32_t* sel_out, void* stream);

/* Dense softmax attention over every cached key, for comparison with the
 * sparse paths: the "Full Attention" column of the ReTopK paper's Table 1
 * (Experimental Results) and Figure 9 (Kernel efficiency analysis). For every
 * (b, h): e_i = q.k_i / sqrt(D) for all i < length (Eq. 4) and
 * out = sum_i softmax(e)_i v_i (Eq. 12 with every position as the support).
 * The row range is split into slices per KV group; the slices' partial
 * results (maximum, weight sum, weighted value sum) are merged as disjoint
 * partial softmax results are (RetrievalAttention reading notes, Method,
 * CPU-GPU two-path computation). Uses the handle's dimensions and its
 * partials workspace; the query-support cache is neither read nor changed.
 * q [B, Hq, D], k and v [B, Hkv, Lmax, D] bf16 (rows 0 .. length-1 are read),
 * out [B, Hq, D] float32. Needs Hq / Hkv <= 8. Two launches on `stream`
 * (slices, then merge); asynchronous, no allocation.
 * Errors: RETOPK_INVALID_ARG for a NULL or misaligned tensor,
 * RETOPK_OUT_OF_RANGE for length outside 1 .. Lmax or more than 8 query heads
 * per KV head, RETOPK_HIP_ERROR when a launch fails. */
retopk_status retopk_dense_attn(retopk_handle* h, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, int32_t length, float* out, void* stream);

/* ---- Several layers: shared workspaces and a graph-replayed decode token ----
 *
 * A decoder runs one decode step per attention layer for every token; the
 * ReTopK paper measures its kernels over the 28 layers of a token and lists
 * per-layer workspace reuse among its kernel stages (Experiments, Kernel
 * efficiency analysis, Table 4). A group holds n_layers handles (one per
 * layer: its own query-support caches and statistics ring) that share ONE set
 * of per-call workspaces (scores, histograms, survivors, candidates, flags),
 * so a layer's memory beyond its caches is not repeated n_layers times. The
 * layers' calls must then be serialised on one stream (they share the
 * workspaces); the per-call outputs that retopk_read_step_info returns are
 * those of the group's most recent call, on whichever layer; the device error
 * word is the group's. Every per-handle entry point works on a layer handle
 * (retopk_group_layer); retopk_destroy ignores layer handles. */
typedef struct retopk_group retopk_group;

/* Create n_layers (1 .. 1024) layers with the parameters *params on the
 * current device, caches empty. Synchronous. *out is NULL on failure. */
retopk_status retopk_group_create(const retopk_params* params, int32_t n_layers, retopk_group** out);

/* Free the group, its layers, workspaces and graph (synchronises the device).
 * A NULL group is ignored. */
void retopk_group_destroy(retopk_group* g);

/* The handle of layer `layer` (0 .. n_layers-1), owned by the group; NULL when
 * out of range. */
retopk_handle* retopk_group_layer(retopk_group* g, int32_t layer);

/* Bytes of device memory the group holds (all layers and the shared workspaces). */
size_t retopk_group_device_bytes(const retopk_group* g);

/* Capture one decode token as a HIP graph owned by the group: a one-thread
 * kernel that moves the group's device position words on by one token
 * (length + 1, t_dec + 1, call sequence + n_layers), then retopk_decode_step
 * of every layer l in order on q[l], k[l], v[l] -> out[l] (arrays of n_layers
 * device pointers, shapes as for retopk_decode_step), each reading its visible
 * length, decode step and call flag from those words instead of from
 * arguments, so that one graph serves every token. Launches are sized for
 * length = max_len. The pointers are fixed in the graph: the caller writes each
 * token's queries (and the new key and value rows) into the same buffers before
 * a replay. `stream` must be a created stream (not NULL); nothing runs during
 * capture. A new capture replaces the previous graph. */
retopk_status retopk_group_capture(retopk_group* g, const uint16_t* const* q, const uint16_t* const* k,
                                   const uint16_t* const* v, float* const* out, void* stream);

/* Position of the next replayed token: visible length `length` (1 .. max_len)
 * and decode step t_dec (>= 1). Host-side only; applied by the next replay. */
retopk_status retopk_group_set_position(retopk_group* g, int32_t length, int32_t t_dec);

/* Replay the captured token on `stream` (one graph launch, plus a one-thread
 * kernel that sets the position words first when the position was just set or
 * eager calls ran on the group since the last replay), then advance the
 * position by one. The same results as retopk_decode_step of every layer in
 * order at that position. Errors: RETOPK_INVALID_ARG when nothing was captured
 * or no position was set; RETOPK_OUT_OF_RANGE when the length would exceed
 * max_len; RETOPK_HIP_ERROR when a launch fails. */
retopk_status retopk_group_replay(retopk_group* g, void* stream);

/* retopk_dense_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * handle, no allocation of any kind. The shapes are given per call (head
 * dimension 128); q, k, v and out are as for retopk_dense_attn, and so is the
 * result, from the same kernels. The row slices' partial results go to a
 * scratch array of 4 MiB that the library holds in device memory on every GPU
 * it runs on until the process ends; a call needs
 * batch * n_q_heads * ceil(CUs / (batch * n_kv_heads)) * 528 bytes of it
 * (0.9 MiB for 28 query heads over 4 KV heads at batch 1 on 256 CUs) and is
 * refused with RETOPK_OUT_OF_RANGE, before any device work, when that exceeds
 * 4 MiB. Every call on one GPU shares that GPU's array: calls that overlap on
 * one GPU (other streams, other threads) race and give wrong results; a call
 * leaves nothing in it that a later call relies on. Uses the current device;
 * two launches on `stream`, asynchronous.
 * Errors: RETOPK_INVALID_ARG for a NULL or misaligned tensor or inconsistent
 * head counts, RETOPK_OUT_OF_RANGE for sizes outside the limits above,
 * RETOPK_NO_DEVICE without a usable GPU, RETOPK_HIP_ERROR when a launch
 * fails. */
retopk_status retopk_dense_attn_noalloc(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t max_len, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, int32_t length, float* out,
                                        void* stream);

/* Copy the caches to host buffers, entries oldest first; unused slots zero.
 *   qbar      float32 [B, Hq, C, D]   normalised queries
 *   supp      int32   [B, Hq, C, K]   supports (ascending), padded with 0
 *   supp_len  int32   [B, Hq, C]      support sizes
 *   count     int32   [B, Hq]         entries held (<= C)
 * Synchronises the device (a test and checkpoint facility, not for the step
 * loop). */
retopk_status retopk_read_state(retopk_handle* h, float* qbar, int32_t* supp,
                                int32_t* supp_len, int32_t* count);

/* Replace the caches from host buffers in the retopk_read_state layout
 * (resume from a snapshot). Each count must be 0 .. C, each supp_len 0 .. K,
 * each support strictly ascending (RETOPK_INVALID_ARG otherwise) with entries
 * 0 .. Lmax-1 (RETOPK_OUT_OF_RANGE otherwise). Synchronous.
 * A later decode step at visible length L ignores stored support entries
 * >= L (those keys are not visible yet, so they cannot be candidates; a
 * library-written cache never holds any, since L never decreases). When a
 * reuse head is left with no candidate at all (W = 0 and nothing visible
 * in the retrieved supports), its support is empty, its output the zero
 * vector, and the pushed entry has support size 0. */
retopk_status retopk_write_state(retopk_handle* h, const float* qbar, const int32_t* supp,
                                 const int32_t* supp_len, const int32_t* count);

/* Copy the decisions of the most recent retopk_decode_step (or exact call) to
 * host buffers. Any pointer may be NULL to skip that field. Synchronises.
 *   path        int32   [B, Hq]          1 = exact, 0 = reuse
 *   rho_max     double  [B, Hq]          -inf when the cache was empty
 *   retrieved   int32   [B, Hq, R]       FIFO positions (0 = oldest) of the
 *                                        retrieved entries, best first, -1 pad
 *   n_cand      int32   [B, Hq]          M_t (0 on exact heads)
 *   cand        int32   [B, Hq, R*K+W]   A_t ascending, first n_cand valid
 *   sel         int32   [B, Hq, K]       S_hat_t ascending, first sel_len valid
 *   sel_len     int32   [B, Hq]
 *   sel_scores  float   [B, Hq, K]       unscaled q.k of the selected keys */
retopk_status retopk_read_step_info(retopk_handle* h, int32_t* path, double* rho_max,
                                    int32_t* retrieved, int32_t* n_cand, int32_t* cand,
                                    int32_t* sel, int32_t* sel_len, float* sel_scores);

/* Statistics ring: per decode step and head, the path (bit 0: exact, bit 1:
 * scheduled refresh), rho_max and M_t. Reads n_steps consecutive steps
 * starting at decode offset first_t_dec (>= 1) into host buffers
 * path [n_steps, B, Hq], rho_max [n_steps, B, Hq], n_cand [n_steps, B, Hq].
 * n_steps <= 4096. Synchronises. Recording is on by default. */
retopk_status retopk_read_stats(retopk_handle* h, int32_t first_t_dec, int32_t n_steps,
                                uint8_t* path, double* rho_max, int32_t* n_cand);
retopk_status retopk_set_stats(retopk_handle* h, int32_t enabled);

/* Kernel timing: when enabled, every kernel launch of the handle is bracketed
 * by HIP events recorded on the launch stream. retopk_read_kernel_times
 * synchronises, accumulates the elapsed time of every recorded launch per
 * kernel, writes total milliseconds and launch counts for kernel ids
 * 0 .. n-1 (n <= retopk_kernel_count()), and clears the record. Up to 65536
 * launches are kept between reads; later ones are not timed. */
retopk_status retopk_set_timing(retopk_handle* h, int32_t enabled);
retopk_status retopk_read_kernel_times(retopk_handle* h, int32_t n, double* total_ms,
                                       int64_t* launches);
int32_t retopk_kernel_count(void);
const char* retopk_kernel_name(int32_t id);

/* Measurement aid, not part of the method: one kernel that reads `bytes`
 * bytes of device memory at `buf` once, as fast as it can, and computes
 * nothing else (the measured streaming-read ceiling beside which the
 * attention kernels' HBM rates are reported). buf must be 16-byte aligned and
 * bytes a multiple of 16; sink is one device uint32 the kernel may write.
 * Uses the current device; asynchronous on `stream`. Errors:
 * RETOPK_INVALID_ARG for a NULL or misaligned pointer or a bad size,
 * RETOPK_HIP_ERROR when the launch fails. */
retopk_status retopk_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Measurement aid, not part of the method: the full-history score pass of
 * one KV group, q.k of 7 query heads (q: 7 rows of 128 bf16) against n_rows
 * key rows (k: [n_rows, 128] bf16, row-major), written once on the matrix
 * cores (use_mfma = 1: 16x16x32 bf16 MFMA tiles) and once on the vector ALUs
 * (use_mfma = 0: bf16 pair dot products), with the same row streaming and
 * grid (one work group per compute unit); the scores are reduced to a
 * running maximum and not stored. Times the choice of unit for the scoring
 * inner loop of retopk_exact_topk_attn. sink is one device float the kernel
 * may write. Uses the current device; asynchronous on `stream`. Errors:
 * RETOPK_INVALID_ARG for a NULL or misaligned pointer or use_mfma not 0/1,
 * RETOPK_OUT_OF_RANGE for n_rows outside 1 .. 2^30, RETOPK_HIP_ERROR when the launch
 * fails. */
retopk_status retopk_score_probe(int32_t use_mfma, const uint16_t* k, int64_t n_rows, const uint16_t* q,
                                 float* sink, void* stream);

/* Bytes of device memory the handle holds. */
size_t retopk_device_bytes(const retopk_handle* h);

/* Sticky device error word of the handle: 0 when every call since the last
 * read completed its work; 1 when a work group of some call gave up one of
 * its bounded waits inside the step (for the path decisions of the call's
 * head work groups, or for other work groups' scores or survivors of an exact
 * KV group), in which case that call's exact heads were not finished and its
 * results are not valid. Synchronises the device, writes the word to *word
 * and clears it. */
retopk_status retopk_read_device_error(retopk_handle* h, int32_t* word);

#ifdef __cplusplus
}
#endif

#endif /* RETOPK_H */
