/*
 * o1.h -- C ABI of the MI355X (gfx950) streaming Nystrom attention library.
 *
 * The operator is the streaming per-GQA-group Nystrom attention of the docs.rs
 * source page of cortiq_engine/nystrom.rs (cortiq-engine 0.5.71): an exact
 * window of the last w keys plus `sink` permanent keys, and a landmark far field
 * sharing one joint denominator (module doc of that page).  This library holds
 * the state of many independent groups -- n_seq sequences x n_layer layers x
 * n_kv KV heads, each KV group serving hpk query heads -- in device memory and
 * advances all of them with one kernel launch per decode step.
 *
 * Conventions for every entry point:
 *   - Tensors are f32, row-major, contiguous, in DEVICE memory owned by the
 *     caller, unless stated otherwise.  The library never frees them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it asynchronously; nothing synchronises with the host.
 *   - Group index g = (s * n_layer + l) * n_kv + kv; the hpk query heads of a
 *     group are contiguous (head h of a model belongs to KV group h / hpk, as in
 *     LayerKvCache::o1_step on the docs.rs LayerKvCache page).
 *   - Return value 0 (O1_OK) on success, otherwise an O1_E* code; the
 *     thread-local o1_last_error() then describes the failure.  A failed call
 *     leaves the state as it was, except O1_EHIP after a launch (state undefined).
 *   - Calls on one handle must be serialised by the caller (one stream, or
 *     external ordering).  Distinct handles are independent.
 *   - A handle lives on the device that was current at o1_create_groups; its
 *     entry points switch to that device for their duration and restore the
 *     caller's current device before returning.
 */
#ifndef O1_H
#define O1_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define O1_ABI_VERSION 3

enum o1_status {
    O1_OK = 0,
    O1_EINVAL = 1,       /* bad argument: null pointer, size or setting out of range */
    O1_ESTATE = 2,       /* call not valid in this state (e.g. step before prefill)  */
    O1_EEXACT = 3,       /* exact-only prompt on a handle created with exact_cap 0   */
    O1_ENOMEM = 4,       /* device allocation failed                                 */
    O1_EHIP = 5,         /* a HIP runtime call or kernel launch failed                */
    O1_EUNSUPPORTED = 6, /* valid for the method but not compiled into this library  */
    O1_EFULL = 7         /* an exact-only group would exceed exact_cap keys           */
};

/* The decode step keeps the value row and per-landmark logits of up to
 * O1_FOLD_PERIOD - 1 evicted keys apart from each head's far numerator T^
 * (NystromHead::far_insert on the nystrom.rs source page adds every evicted key
 * to T^ at once) and adds them all to T^ with every O1_FOLD_PERIOD-th eviction,
 * so T^, otherwise the step's largest write, is rewritten once per
 * O1_FOLD_PERIOD steps.  With w >= O1_FOLD_PERIOD the far-insert logits
 * q~ . k * scale of each key are computed on the fold that follows its arrival
 * (one pass over q~ per O1_FOLD_PERIOD steps) and kept with its ring slot until
 * it leaves.  Outputs are those of the per-eviction update up to rounding.  A
 * group's held count is its far_len mod O1_FOLD_PERIOD. */
#define O1_FOLD_PERIOD 8

/* O1Rect of the nystrom.rs source page: how the indefinite skeleton is
 * rectified.  AGGREGATE (the page's default) drops a row's far field when its
 * far denominator is negative; FM clamps the mixing row u = F M at zero. */
enum o1_rect { O1_RECT_AGGREGATE = 0, O1_RECT_FM = 1 };

/* Geometry of a batch of groups (NystromState::new_group on the nystrom.rs
 * source page: m >= 4, w >= 1, q_heads >= 1).  Defaults on that page:
 * m = 32, w = 128, sink = 4, rect = AGGREGATE.
 * Compiled shapes: d == dv in {64, 80, 96, 128, 256} or d = 192 with dv = 128
 * (keys wider than values), hpk <= 64, m <= 64, sink + w <= 4096 with
 * hpk' * (sink + w) <= 4096, hpk' being min(hpk, B) rounded up to a power of
 * two, B = 8 heads per block (4 at d = 80) (the kernels for hpk' heads run the
 * groups of hpk' / 2 < hpk <= hpk' heads; a group of more than B heads is
 * stepped in blocks of at most B heads, one launch each, on the caller's
 * stream); other valid shapes return O1_EUNSUPPORTED.
 *
 * exact_cap sizes the exact-only mode (NystromGroup::prefill_shared on the
 * nystrom.rs source page): a prompt of T <= w + sink + 8 tokens builds no
 * skeleton; the group keeps every key exactly and each decode step appends one,
 * so the window grows without bound on that page.  Here it grows into buffers
 * of exact_cap keys per group, allocated once by o1_create_groups; 0 allocates
 * nothing and such prompts return O1_EEXACT.
 *
 * ridge_rel is the relative ridge of the mixing matrix's pseudo-inverse
 * (RIDGE_REL = 1e-6 on the nystrom.rs source page, used when it is 0):
 * lambda = ridge_rel * max(mean diag(A^T A), DBL_MIN).  Other values exist to
 * test the retry path of ridge_pinv (lambda grown tenfold after a failed
 * Cholesky factorisation); a model has no reason to set it. */
typedef struct o1_config {
    int32_t n_seq;    /* sequences                         (>= 1) */
    int32_t n_layer;  /* layers per sequence               (>= 1) */
    int32_t n_kv;     /* KV heads (groups) per layer       (>= 1) */
    int32_t hpk;      /* query heads per KV group          (>= 1) */
    int32_t d;        /* query / key width                 (>= 1) */
    int32_t dv;       /* value width                       (>= 1) */
    int32_t m;        /* landmark budget                   (>= 4) */
    int32_t w;        /* exact window width                (>= 1) */
    int32_t sink;     /* permanent exact sink keys         (>= 0) */
    int32_t rect;     /* enum o1_rect                             */
    int32_t exact_cap;/* keys an exact-only group may hold   (>= 0) */
    double ridge_rel; /* 0 = 1e-6; otherwise finite, > 0           */
} o1_config;

typedef struct o1_groups o1_groups; /* opaque; owns every state buffer */

/* Optional replacements for the frozen landmarks and mixing matrix of a
 * prefill (device pointers, f32; NULL = compute as the page does):
 *   k_tilde [G][m_eff][d], q_tilde [G][hpk][m_eff][d],
 *   mu      [G][hpk][m_eff][m_eff]  (row a = key landmark, column b = query
 *                                    landmark, as NystromHead::step reads it).
 * A replaced k_tilde / q_tilde also feeds the exp-Gram of a computed mu. */
typedef struct o1_frozen {
    const float *k_tilde;
    const float *q_tilde;
    const float *mu;
} o1_frozen;

typedef struct o1_info {
    int32_t n_groups;     /* G = n_seq * n_layer * n_kv                         */
    int32_t sealed;       /* 1 when every layer has a successful prefill         */
    int32_t prompt_len;   /* T of the sealed layers (0 when none is)             */
    int32_t m_eff;        /* clamp(T / 8, 4, m); 0 when none is sealed or exact-only */
    int64_t steps;        /* decode steps of the least advanced sealed layer     */
    uint64_t state_bytes; /* device bytes of the persistent per-group state      */
    uint64_t work_bytes;  /* device bytes of prefill work buffers currently held */
    int32_t exact_only;   /* 1 when the sealed prompt took the exact-only mode   */
    int32_t exact_keys;   /* keys held exactly per group: sink + w, or, exact-only,
                             T + max_steps (the fullest layer)                   */
    int32_t n_layer;      /* layers per sequence                                 */
    int32_t layers_sealed;/* layers with a successful prefill of the prompt      */
    int64_t max_steps;    /* decode steps of the most advanced sealed layer      */
    /* NystromState::memory_bytes of the nystrom.rs source page, summed over the
     * groups of the sealed layers: the f32 words of the vectors the page keeps
     * per group (window w (d + dv), sinks sink (d + dv), K~ m d) and per head
     * (T^ m dv, Z^ m, running max m, Q~ m d, M m m, score scratch sink + w and
     * three m-long scratch vectors), times 4.  In the exact-only mode a group
     * counts its keys, n (d + dv), and each head a score scratch of n entries
     * once the layer has stepped (none before).  Steps are counted per call, as
     * `steps` is.  This is the page's figure, not this library's allocation. */
    uint64_t page_bytes;
    uint64_t fold_bytes;       /* device bytes of the held evictions (value rows, their
                                  logits, T^'s scale): part of state_bytes, not on the page */
    uint64_t ring_logit_bytes; /* device bytes of the far-insert logits kept per ring
                                  slot (0 when w < O1_FOLD_PERIOD): part of state_bytes */
    /* The ridge of every head of the sealed skeleton-mode layers whose M was
     * computed (not given as frozen): smallest, median and largest lambda, the
     * largest Cholesky attempt number (13 = the scaled-identity fallback), and
     * the heads that needed more than one attempt / took the fallback.  All 0
     * when no such head exists. */
    double lambda_min, lambda_median, lambda_max;
    int32_t tries_max;
    int32_t heads_retried;
    int32_t heads_fallback;
    int32_t ridge_heads;       /* heads these figures cover                           */
} o1_info;

/* Fields of the device state, for o1_field_bytes / o1_read_field /
 * o1_write_field.  Shapes use G groups, R = sink + w near rows, m = m_eff.
 * near_k/near_v rows 0..sink-1 are the sinks, row sink + s is ring slot s. */
enum o1_field {
    O1_FIELD_NEAR_K = 0,   /* f32 [G][R][d]                                    */
    O1_FIELD_NEAR_V = 1,   /* f32 [G][R][dv]                                   */
    O1_FIELD_K_TILDE = 2,  /* f32 [G][m][d]       key landmarks                */
    O1_FIELD_Q_TILDE = 3,  /* f32 [G][hpk][m][d]  query landmarks              */
    O1_FIELD_MU = 4,       /* f32 [G][hpk][m][m]  mixing matrix M              */
    O1_FIELD_T_HAT = 5,    /* f32 [G][hpk][m][dv] far numerator at e^{-m_max}  */
    O1_FIELD_Z_HAT = 6,    /* f64 [G][hpk][m]     far denominator at e^{-m_max} */
    O1_FIELD_M_MAX = 7,    /* f32 [G][hpk][m]     per-landmark running max     */
    O1_FIELD_WIN_HEAD = 8, /* i32 [G]             ring slot of the oldest key  */
    O1_FIELD_FAR_LEN = 9,  /* i64 [G][hpk]        keys absorbed per head       */
    O1_FIELD_LAMBDA = 10,  /* f64 [G][hpk]        ridge used by the pinv       */
    O1_FIELD_TRIES = 11,   /* i32 [G][hpk]        Cholesky attempt that worked (13 = fallback) */
    O1_FIELD_EXACT_K = 12, /* f32 [G][exact_cap][d]  exact-only keys, row j = position j   */
    O1_FIELD_EXACT_V = 13, /* f32 [G][exact_cap][dv] exact-only values                     */
    O1_FIELD_COUNT = 14
};

/* Validate `cfg` and allocate the state of all its groups on the current HIP
 * device (once; decode never allocates).  *out receives the handle.
 * Errors: O1_EINVAL (null pointer, m < 4, w < 1, hpk < 1, sink < 0, d or dv
 * < 1, counts < 1, unknown rect, exact_cap < 0 or too large), O1_EUNSUPPORTED,
 * O1_ENOMEM, O1_EHIP. */
int o1_create_groups(const o1_config *cfg, o1_groups **out);

/* Release every buffer of the handle.  NULL is a no-op.  The caller must make
 * sure no work using the handle is still pending. */
void o1_destroy_groups(o1_groups *g);

/* Prefill freeze (NystromState::prefill_group, NystromGroup::prefill_shared and
 * NystromHead::seal on the nystrom.rs source page) for every group at once:
 *   q [G][hpk][T][d]   each head's prompt queries
 *   k [G][T][d]        the group's prompt keys
 *   v [G][T][dv]       the group's prompt values
 * Sets the sinks (rows 0..sink-1), the ring (the last w keys, key j in slot
 * (j - sink) mod w), m_eff = clamp(T/8, 4, m), K~ and each head's Q~ as segment
 * means (f64 accumulation, stored f32), M = ridge pinv of exp(Q~ K~^T / sqrt d)
 * in f64 (lambda = 1e-6 mean diag(A^T A), grown tenfold on a failed Cholesky,
 * up to 12 times), and the far field of keys sink .. T-w-1 (T^, Z^, running
 * max, far_len = T - sink - w).  `frozen` may be NULL.  Resets any earlier
 * state of the handle.
 * A prompt of T <= w + sink + 8 tokens takes the exact-only mode instead: the
 * T keys and values become rows 0 .. T-1 of the group's exact buffers, there
 * are no sinks, landmarks or far field (m_eff = 0, far_len = 0), and `q`
 * (which may then be NULL) and `frozen` are not read.
 * Every tensor must be 16-byte aligned.
 * Errors: O1_EINVAL (null or misaligned tensor, T < 1, T * G * hpk * d > 2^40),
 * O1_EEXACT (exact-only prompt and exact_cap = 0), O1_EFULL (exact-only prompt
 * longer than exact_cap), O1_ENOMEM (work buffers), O1_EHIP. */
int o1_prefill(o1_groups *g, const float *q, const float *k, const float *v, int32_t T,
               const o1_frozen *frozen, void *stream);

/* One decode step (NystromState::step_group on the nystrom.rs source page) for
 * every group: insert the group's new key/value once, absorb the key leaving
 * the window into every head's far field, and write every head's output.
 *   q   [G][hpk][d]    queries of the new position
 *   k   [G][d], v [G][dv]  the new key / value
 *   out [G][hpk][dv]   outputs (may not alias the inputs)
 * In the exact-only mode the step appends (k, v) as key n = T + steps and
 * writes, per head, softmax attention over keys 0 .. n (NystromHead::step with
 * no sinks and no far field).  Each group's key count is kept on the device
 * and advanced by the step itself, so layers stepped one by one to different
 * counts are stepped correctly by o1_step as well.  Launches: the attention,
 * plus a merge when a group's keys are split across work-groups.
 * No allocation, no host synchronisation; one kernel launch in the skeleton
 * mode.
 * Graph capture: a step (and o1_step_layer) may be captured into a HIP graph
 * and replayed, in either mode; each replay advances the device state as a
 * call does.  The step counts o1_get_info reports count calls only.  A replay
 * that finds an exact-only group already holding exact_cap keys changes
 * nothing for that group and writes none of its outputs (an eager call
 * returns O1_EFULL instead).
 * Errors: O1_EINVAL (null or misaligned tensor), O1_ESTATE (a layer without a
 * successful prefill), O1_EFULL (exact-only group already holding exact_cap
 * keys; nothing is changed), O1_EHIP. */
int o1_step(o1_groups *g, const float *q, const float *k, const float *v, float *out,
            void *stream);

/* ---- one layer at a time, from a model's own buffers ----------------------
 * A model seals each layer at the end of its exact prompt pass and then steps
 * it once per token (LayerKvCache::o1_begin / o1_push_q / o1_seal / o1_step on
 * the docs.rs LayerKvCache page).  These two entry points cover the groups of
 * one layer l of every sequence -- groups (s * n_layer + l) * n_kv + kv -- and
 * read the prompt in place.
 *
 * The prompt of one layer, as element strides (in floats).  For sequence s, KV
 * head kv, query head j of that group (model head kv * hpk + j), position t
 * and component c:
 *   q[s * q_seq + (kv * hpk + j) * q_head + t * q_pos + c]
 *   k[s * k_seq + kv * k_kv + t * k_pos + c],   v likewise with v_*.
 * Rows are contiguous; every stride is a non-negative multiple of 4 and every
 * pointer 16-byte aligned.  Examples: the query trace o1_push_q collects,
 * [n_seq][T][n_kv * hpk][d], has q_seq = T * n_kv * hpk * d, q_head = d,
 * q_pos = n_kv * hpk * d; per-KV-head caches [n_seq][n_kv][cap][d] (the page's
 * k_heads / v_heads) have k_seq = n_kv * cap * d, k_kv = cap * d, k_pos = d. */
typedef struct o1_prompt_view {
    const float *q;
    int64_t q_seq, q_head, q_pos;
    const float *k;
    int64_t k_seq, k_kv, k_pos;
    const float *v;
    int64_t v_seq, v_kv, v_pos;
} o1_prompt_view;

/* Prefill freeze of layer `layer` of every sequence, as o1_prefill does for
 * the whole handle (same steps, modes and errors), reading the first T
 * positions of `p`.  `frozen` arrays, if given, cover the layer's groups in
 * the order (s, kv).  Every layer of a handle shares one prompt length: a
 * layer prefill with a T other than the sealed layers' starts a new prompt
 * and leaves the other layers unsealed until they are sealed again.
 * Errors: those of o1_prefill; O1_EINVAL also for a layer out of range, a
 * misaligned pointer or a bad stride. */
int o1_prefill_layer(o1_groups *g, int32_t layer, const o1_prompt_view *p, int32_t T,
                     const o1_frozen *frozen, void *stream);

/* One decode step of layer `layer` of every sequence (LayerKvCache::o1_step):
 *   q   [n_seq][n_kv * hpk][d]   the layer's queries, model head order
 *   k   [n_seq][n_kv][d], v [n_seq][n_kv][dv]
 *   out [n_seq][n_kv * hpk][dv]
 * One launch, as o1_step; the layer's step count advances by one.
 * Errors: O1_EINVAL (null or misaligned tensor, layer out of range),
 * O1_ESTATE (layer not sealed), O1_EFULL (exact-only layer holding exact_cap
 * keys), O1_EHIP. */
int o1_step_layer(o1_groups *g, int32_t layer, const float *q, const float *k, const float *v,
                  float *out, void *stream);

/* Facts about the handle.  The ridge figures are read from the device: the
 * first call after a prefill (or a write of O1_FIELD_LAMBDA / O1_FIELD_TRIES)
 * waits for the device to finish its work (hipDeviceSynchronize) and copies
 * every head's lambda and attempt number to the host; later calls reuse that
 * copy and do no device work.  Not to be called while a stream of the
 * device is being captured.  Errors: O1_EINVAL, O1_EHIP. */
int o1_get_info(const o1_groups *g, o1_info *info);

/* Bytes of one state field at the current m_eff (see enum o1_field).
 * Errors: O1_EINVAL (unknown field, null pointer, exact buffers of a handle
 * created with exact_cap = 0), O1_ESTATE (landmark-shaped fields before a
 * skeleton prefill, or in the exact-only mode). */
int o1_field_bytes(const o1_groups *g, int32_t field, size_t *bytes);

/* Copy a whole state field to `dst` / from `src` (host or device memory;
 * `bytes` must equal o1_field_bytes), enqueued on `stream`.  For tests and
 * state transfer; the decode path never needs them.  Reading O1_FIELD_T_HAT
 * returns T^ with the held evictions (O1_FOLD_PERIOD) added, built in a
 * stream-ordered temporary; the state is left as it is.  Every write first
 * adds the held evictions to the stored T^ (none are held afterwards), a
 * write of O1_FIELD_M_MAX takes the stored T^ to be at the new running max, and
 * every write recomputes the far-insert logits of all keys in the ring (a write
 * may change the ring's keys, q~, or the counters that schedule the folds that
 * would otherwise compute them).
 * Writing requires a sealed layer.
 * Errors: O1_EINVAL, O1_ESTATE, O1_ENOMEM (the T^ temporary), O1_EHIP. */
int o1_read_field(const o1_groups *g, int32_t field, void *dst, size_t bytes, void *stream);
int o1_write_field(o1_groups *g, int32_t field, const void *src, size_t bytes, void *stream);

/* ---- exact grouped-GQA attention: the O(p) comparator -------------------
 * Exact softmax attention of every query head of a KV group over that group's
 * stored keys (LayerKvCache::attend_group on the docs.rs LayerKvCache page:
 * one pass over the K rows and one over the V rows for all heads of a group;
 * keys before `first` get zero probability):
 *   out[g][h] = sum_{j = first .. n_keys-1} softmax_j(q[g][h] . k[g][j] * scale) v[g][j]
 * The caller owns the cache; nothing is stored between calls.  q8 storage,
 * logit soft-capping and the importance accumulator of that method are not
 * part of this entry point. */
typedef struct o1_exact_desc {
    int32_t n_groups; /* G                                        (>= 1)      */
    int32_t hpk;      /* query heads per group                   1 .. 64     */
    int32_t d, dv;    /* widths: d == dv in {64, 80, 96, 128, 256}, or 192/128 */
    int32_t cap;      /* rows allocated per group (row stride of k and v)   */
    int32_t first;    /* earliest visible key, 0 <= first < n_keys          */
    int32_t n_keys;   /* keys 0 .. n_keys-1 are stored, n_keys <= cap       */
    float scale;      /* score scale; <= 0 selects f32 1/sqrt(d)            */
} o1_exact_desc;

/* Bytes of device work space o1_exact_attend needs for `desc` (0 when it
 * needs none).  Errors: O1_EINVAL, O1_EUNSUPPORTED. */
int o1_exact_workspace_bytes(const o1_exact_desc *desc, size_t *bytes);

/* Exact attention for all G groups in one launch (two when the key range is
 * split across work-groups):
 *   q [G][hpk][d], k [G][cap][d], v [G][cap][dv] -> out [G][hpk][dv]
 * `workspace` (device, caller-owned) must hold o1_exact_workspace_bytes; it
 * may be NULL when that is 0.  No allocation, no host synchronisation.
 * Errors: O1_EINVAL (null pointer, bad sizes, short work space),
 * O1_EUNSUPPORTED, O1_EHIP. */
int o1_exact_attend(const o1_exact_desc *desc, const float *q, const float *k, const float *v,
                    float *out, void *workspace, size_t workspace_bytes, void *stream);

/* o1_exact_attend for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results, without the work space: the split
 * partials go to a static buffer of O1_EXACT_NOALLOC_BYTES in the library's
 * device memory, one per device, held until the process ends (its device
 * address is looked up on the first call on each device).  Nothing is
 * allocated, by the library or by the caller.
 * Every call on a device shares that device's buffer: calls that may run at
 * the same time on one device (different streams, or graphs replayed
 * concurrently) race on it and must be ordered by the caller.
 * Errors: those of o1_exact_attend; O1_EINVAL also when the launch needs more
 * work space than the buffer holds (o1_exact_workspace_bytes of `desc` above
 * O1_EXACT_NOALLOC_BYTES; then use o1_exact_attend). */
#define O1_EXACT_NOALLOC_BYTES (16u << 20)
int o1_exact_attend_noalloc(const o1_exact_desc *desc, const float *q, const float *k, const float *v,
                            float *out, void *stream);

/* Description of the last failure on the calling thread ("" if none). */
const char *o1_last_error(void);

/* O1_ABI_VERSION of the library. */
int o1_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* O1_H */
