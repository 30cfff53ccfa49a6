// Internal interface between the C-ABI host code (o1_api.hip) and the gfx950
// kernels (o1_decode.hip, o1_prefill.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "o1.h"

namespace o1 {

constexpr int kMaxLandmarks = 64;      // largest m_eff the kernels are compiled for
constexpr double kDenEps = 1e-30;      // DEN_EPS of the nystrom.rs source page
constexpr double kRidgeRel = 1e-6;     // RIDGE_REL of the nystrom.rs source page
constexpr int kRidgeTries = 12;        // ridge_pinv: attempts before the fallback
constexpr int kExactSlack = 8;         // EXACT_SLACK of the nystrom.rs source page
constexpr size_t kInfinityCacheBytes = size_t(256) << 20;  // MI355X memory-side cache
// Evictions held apart from T^: the value row and per-landmark logits of up to
// kPend - 1 evicted keys wait in small per-group buffers, and every kPend-th
// eviction folds them all into T^ at once, so T^ is rewritten once per kPend
// steps instead of every step.  A group's held count is far_len mod kPend.
constexpr int kPend = O1_FOLD_PERIOD;

// Largest power of two not above `want` that divides n; smallest power of two
// not below n; largest power of two not above n (n >= 1).
__host__ __device__ constexpr int pow2_divisor(int want, int n)
{
    int p = 1;
    while (2 * p <= want && n % (2 * p) == 0) p *= 2;
    return p;
}
__host__ __device__ constexpr int pow2_ceil(int n)
{
    int p = 1;
    while (p < n) p *= 2;
    return p;
}
__host__ __device__ constexpr int pow2_floor(int n)
{
    int p = 1;
    while (2 * p <= n) p *= 2;
    return p;
}
static_assert(kPend >= 2, "a fold period of 1 holds nothing");

// Device state of G independent groups (one GQA group each).  Layout, with
// R = sink + w near rows and m = m_eff:
//   near_k [G][R][d], near_v [G][R][dv]   rows 0..sink-1 sinks, row sink+s ring slot s
//   k_tilde [G][m][d]                     key landmarks (f32)
//   q_tilde [G][hpk][m][d]                query landmarks (f32)
//   mu      [G][hpk][m][m]                mixing matrix, row = key landmark
//   t_hat   [G][hpk][m][dv] (f32), z_hat [G][hpk][m] (f64), m_max [G][hpk][m] (f32)
//   win_head [G] (i32), far_len [G][hpk] (i64), lambda [G][hpk] (f64), tries [G][hpk] (i32)
// Held evictions (see kPend): with P = far_len mod kPend evictions held,
//   pend_v [G][kPend][dv] (f32)           value rows of the held evictions, slot j < P
//   pend_l [G][hpk][kPend][m] (f64)       their logits q~_i . k * scale (-inf: empty slot)
//   m_ref  [G][hpk][m] (f32)              the running max at the last fold: the stored
//                                         t_hat is at scale e^{-m_ref}; the far numerator is
//   T^_i = e^{m_ref_i - m_max_i} t_hat_i + sum_{j<P} e^{pend_l_ij - m_max_i} pend_v_j
// Far-insert logits of the keys in the ring (only when w >= kPend):
//   ring_l [G][w][hpk][m] (f64)           q~_{h,i} . k * scale for the key in ring slot s,
//                                         computed within kPend steps of the key's arrival
//                                         (one pass over q~ per fold) and read when it leaves
struct DevState {
    int G, hpk, d, dv, w, sink, R, rect;
    int m;        // m_eff of the current prefill
    float scale;  // f32 1/sqrt(d), as NystromGroup::prefill_shared sets it
    float *near_k, *near_v, *k_tilde, *q_tilde, *mu, *t_hat, *m_max;
    double *z_hat, *lambda;
    int32_t *win_head, *tries;
    int64_t *far_len;
    float *pend_v, *m_ref;
    double *pend_l;
    double *ring_l;    // null when w < kPend (the step then reads q~ at every eviction)
    int stream_state;  // 1 when the state is larger than the Infinity Cache (decode streams it)
};

// The groups one call covers.  Its inputs and outputs are indexed by the call's
// own index i in [0, count); state group g = (i / per) * stride + offset + i % per.
//   whole handle:   per = stride = n_kv, offset = 0        (g = i)
//   one layer l:    per = n_kv, stride = n_layer * n_kv, offset = l * n_kv
//                   (i = s * n_kv + kv, the layer's groups of every sequence)
struct GroupMap {
    int count, per, stride, offset;
    __host__ __device__ int state(int i) const { return (i / per) * stride + offset + i % per; }
};

// A prompt in place, element strides in floats.  For call index i (o = i / per,
// n = i % per), query head j of the group, position t and component c:
//   q(i, j, t, c) = q[o * q_outer + (n * hpk + j) * q_head + t * q_pos + c]
//   k(i, t, c)    = k[o * k_outer + n * k_inner + t * k_pos + c]     (v alike)
// Rows are contiguous; strides are multiples of 4 floats (float4 rows).
struct PromptView {
    const float *q, *k, *v;
    int64_t q_outer, q_head, q_pos;
    int64_t k_outer, k_inner, k_pos;
    int64_t v_outer, v_inner, v_pos;
    __host__ __device__ const float *q_row(const GroupMap &mp, int hpk, int i, int j, int64_t t) const
    {
        return q + (int64_t)(i / mp.per) * q_outer + ((int64_t)(i % mp.per) * hpk + j) * q_head + t * q_pos;
    }
    __host__ __device__ const float *k_row(const GroupMap &mp, int i, int64_t t) const
    {
        return k + (int64_t)(i / mp.per) * k_outer + (int64_t)(i % mp.per) * k_inner + t * k_pos;
    }
    __host__ __device__ const float *v_row(const GroupMap &mp, int i, int64_t t) const
    {
        return v + (int64_t)(i / mp.per) * v_outer + (int64_t)(i % mp.per) * v_inner + t * v_pos;
    }
};

// Heads per decode launch: a group of more heads is stepped in blocks of this
// many (the kernels are compiled for 1, 2, 4 and 8 heads), up to kMaxHeads
// query heads per group (a 64-head attention over one KV head).
constexpr int kMaxBlockHeads = 8;
constexpr int kMaxHeads = 64;

// Heads per block at key width d: the row dots split a key row of d/4 float4
// over a power-of-two number of lanes (at most 32 for 8 heads) that must be at
// least the block's head count, so widths whose d/4 has a smaller power-of-two
// factor (d = 80: 20 float4, four lanes of 5) take blocks of fewer heads.
__host__ __device__ constexpr int block_heads(int d)
{
    return pow2_divisor(32, d / 4) < kMaxBlockHeads ? pow2_divisor(32, d / 4) : kMaxBlockHeads;
}

// Key and value widths the kernels are compiled for: d == dv in {64, 80, 96,
// 128, 256}, and keys of 192 floats with values of 128 (a head whose queries
// and keys carry 64 more components than its values).
constexpr bool widths_compiled(int d, int dv)
{
    return (d == dv && (d == 64 || d == 80 || d == 96 || d == 128 || d == 256)) || (d == 192 && dv == 128);
}

struct DecodeIO {
    const float *q, *k, *v;  // q [count][hpk][d], k [count][d], v [count][dv]
    float *out;              // [count][hpk][dv]
    GroupMap map;
    // Heads h0 .. h0 + hb - 1 of every group (a group of more than 8 heads is
    // stepped in blocks of at most 8, one launch each, in order).  `shared`:
    // this launch also makes the group's shared writes (the new row into the
    // ring, the evicted value row into the held set, the ring position), which
    // the last block's launch does after every other block has read the ring.
    int h0 = 0, hb = 0;
    int shared = 1;
};

struct PrefillIO {
    PromptView p;
    GroupMap map;
    int T;
    const float *fz_kt, *fz_qt, *fz_mu;  // optional frozen replacements, [count][...]
    double *a64;                         // work: [count][hpk][mp][mp] f64 exp-Gram of each head, zero past m
    double ridge_rel;                    // relative ridge of the pinv (RIDGE_REL unless a test sets it)
};

// Exact grouped-GQA attention over a stored KV cache: the O(p) comparator, and
// the decode step of the exact-only mode.  q, out, k_new, v_new and the split
// partials are indexed by the call index i, the cache by the state group map.state(i).
struct ExactIO {
    const float *q, *k, *v;  // q [count][hpk][d], k [G][cap][d], v [G][cap][dv]
    float *out;              // [count][hpk][dv]
    GroupMap map;
    int hpk, d, dv, cap, first, n_keys, per_split;
    // Set by launch_exact, which runs a group of more heads than block_heads(d)
    // in blocks: the kernels then see hpk = the block's heads, hg = the
    // group's (the stride of q and out), h0 = the block's first head, and
    // shared = 1 for the last block only, which alone stores the appended
    // key and advances the key count.
    int hg, h0, shared;
    float scale;
    double *ws_max, *ws_sum, *ws_num;  // split partials [count][splits][hpk](x dv)
    // Append mode (exact-only decode), else all null: key n_keys-1 is the new
    // one, read from k_new [count][d] / v_new [count][dv] and stored into row
    // n_keys-1 of k_dst / v_dst (the same buffers as k / v).
    const float *k_new, *v_new;
    float *k_dst, *v_dst;
    // Exact-only decode: keys held per state group, read on the device (so a
    // graph replay sees the current count) -- group g holds held[g] keys and
    // gets n_keys = held[g] + 1 after the append; a group already holding cap
    // keys is left untouched.  The key range of a split is then
    // ceil(n_keys / splits) keys.  The step advances held[g] itself (its one
    // work-group, or the merge of its split ranges).  Null otherwise.
    int32_t *held;
};
int exact_splits(int G, int n_visible);
hipError_t launch_exact(const ExactIO &io, int splits, hipStream_t stream);
// Exact-only prefill of the groups in `map`: prompt rows 0..T-1 into rows
// 0..T-1 of ek [G][cap][d], ev [G][cap][dv]; win_head, far_len, lambda, tries
// cleared; held[g] = T for each mapped group g.
hipError_t launch_exact_seal(const DevState &s, const PromptView &p, const GroupMap &map, int T,
                             float *ek, float *ev, int cap, int32_t *held, hipStream_t stream);

// True when the decode kernel is compiled for this shape.
bool decode_supported(int d, int dv, int hpk, int m, int R);
hipError_t launch_decode(const DevState &s, const DecodeIO &io, hipStream_t stream);
// ring_l of every ring slot of the groups in `map` from their ring rows and q~
// (after a prefill, and after every state write).  No-op when ring_l is null.
hipError_t launch_ring_logits(const DevState &s, const GroupMap &map, hipStream_t stream);
// T^ with the held evictions folded in, for every group, into dst ([G][hpk][m][dv]
// f32; may be s.t_hat).  With `reset` the state's held set is then emptied
// (m_ref = m_max, every slot's logits -inf); dst must then be s.t_hat.
hipError_t launch_fold(const DevState &s, float *dst, bool reset, hipStream_t stream);
hipError_t launch_prefill(const DevState &s, const PrefillIO &io, hipStream_t stream);

// ---- wavefront helpers (wave64) ------------------------------------------
//
// Cross-lane exchanges of f64 values on the vector ALU (no LDS crossbar).
// Within 16-lane rows a partner lane whose lane bit OFF is flipped comes from
// DPP (lane ^ 1 and lane ^ 2 by quad permutes, 7 - i in each 8-lane half row
// and 15 - i in each row by the mirrors).  Across rows and wave halves
// (lane ^ 16, lane ^ 32) v_permlane16_swap / v_permlane32_swap exchange two
// registers at once.  A reduction that pairs every lane with one lane of the
// other half at each level sums every lane exactly once, whichever partner of
// that half it is.
namespace lanes {

__device__ __forceinline__ unsigned lo32(double x) { return (unsigned)__double_as_longlong(x); }
__device__ __forceinline__ unsigned hi32(double x) { return (unsigned)(__double_as_longlong(x) >> 32); }
__device__ __forceinline__ double join(unsigned lo, unsigned hi)
{
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int CTRL>
__device__ __forceinline__ double dpp(double x)
{
    return join((unsigned)__builtin_amdgcn_update_dpp(0, (int)lo32(x), CTRL, 0xf, 0xf, false),
                 (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi32(x), CTRL, 0xf, 0xf, false));
}

}  // namespace lanes

template <int OFF>
__device__ __forceinline__ double partner(double x)
{
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8, "lane bit within a row");
    if constexpr (OFF == 1) {
        return lanes::dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    } else if constexpr (OFF == 2) {
        return lanes::dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    } else if constexpr (OFF == 4) {
        return lanes::dpp<0x141>(x);  // row_half_mirror: 7 - i within 8 lanes
    } else {
        return lanes::dpp<0x140>(x);  // row_mirror: 15 - i within 16 lanes
    }
}

// Halving exchange across 16-lane rows (OFF = 16) or wave halves (OFF = 32):
// lanes with lane bit OFF clear return a + a(lane ^ OFF), lanes with it set
// b + b(lane ^ OFF).  One swap of (a, b) leaves, in every lane, its own kept
// value in one output and its partner's in the other, so no select is needed
// (the sum is exact in either order).
template <int OFF>
__device__ __forceinline__ double swap_sum(double a, double b)
{
    static_assert(OFF == 16 || OFF == 32, "whole-row exchanges only");
    if constexpr (OFF == 16) {
        const auto lo = __builtin_amdgcn_permlane16_swap(lanes::lo32(a), lanes::lo32(b), false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(lanes::hi32(a), lanes::hi32(b), false, false);
        return lanes::join(lo[0], hi[0]) + lanes::join(lo[1], hi[1]);
    } else {
        const auto lo = __builtin_amdgcn_permlane32_swap(lanes::lo32(a), lanes::lo32(b), false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(lanes::hi32(a), lanes::hi32(b), false, false);
        return lanes::join(lo[0], hi[0]) + lanes::join(lo[1], hi[1]);
    }
}

// max(x, x(lane ^ OFF)) for OFF = 16 or 32, from one swap as in swap_sum
template <int OFF>
__device__ __forceinline__ double swap_max(double x)
{
    static_assert(OFF == 16 || OFF == 32, "whole-row exchanges only");
    if constexpr (OFF == 16) {
        const auto lo = __builtin_amdgcn_permlane16_swap(lanes::lo32(x), lanes::lo32(x), false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(lanes::hi32(x), lanes::hi32(x), false, false);
        return fmax(lanes::join(lo[0], hi[0]), lanes::join(lo[1], hi[1]));
    } else {
        const auto lo = __builtin_amdgcn_permlane32_swap(lanes::lo32(x), lanes::lo32(x), false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(lanes::hi32(x), lanes::hi32(x), false, false);
        return fmax(lanes::join(lo[0], hi[0]), lanes::join(lo[1], hi[1]));
    }
}

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of
// the group receives the group total.
template <int W>
__device__ __forceinline__ double group_sum(double x)
{
    if constexpr (W >= 64) x = swap_sum<32>(x, x);
    if constexpr (W >= 32) x = swap_sum<16>(x, x);
    if constexpr (W >= 16) x += partner<8>(x);
    if constexpr (W >= 8) x += partner<4>(x);
    if constexpr (W >= 4) x += partner<2>(x);
    if constexpr (W >= 2) x += partner<1>(x);
    return x;
}

__device__ __forceinline__ double wave_sum(double x) { return group_sum<64>(x); }

__device__ __forceinline__ double wave_max(double x)
{
    x = swap_max<32>(x);
    x = swap_max<16>(x);
    x = fmax(x, partner<8>(x));
    x = fmax(x, partner<4>(x));
    x = fmax(x, partner<2>(x));
    return fmax(x, partner<1>(x));
}

// Max over aligned groups of W lanes within a 16-lane row (W <= 16); every lane
// of the group receives the group maximum.
template <int W>
__device__ __forceinline__ double group_max(double x)
{
    static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "group within a DPP row");
    if constexpr (W >= 16) x = fmax(x, partner<8>(x));
    if constexpr (W >= 8) x = fmax(x, partner<4>(x));
    if constexpr (W >= 4) x = fmax(x, partner<2>(x));
    if constexpr (W >= 2) x = fmax(x, partner<1>(x));
    return x;
}

// Sum over the lanes that differ from this one only in lane bits >= FROM: the
// partners are exact (lane ^ 16, lane ^ 32), so the lower lane bits -- a column
// index, say -- are kept.
template <int FROM>
__device__ __forceinline__ double sum_high_lanes(double x)
{
    static_assert(FROM == 16 || FROM == 32 || FROM == 64, "only whole 16-lane rows are exchanged exactly");
    if constexpr (FROM <= 16) x = swap_sum<16>(x, x);
    if constexpr (FROM <= 32) x = swap_sum<32>(x, x);
    return x;
}

// Value of lane `src` (uniform across the wave) in every lane.
__device__ __forceinline__ double lane_value(double x, int src)
{
    return lanes::join((unsigned)__builtin_amdgcn_readlane((int)lanes::lo32(x), src),
                       (unsigned)__builtin_amdgcn_readlane((int)lanes::hi32(x), src));
}

// ---- row arithmetic shared by the decode and exact-attention kernels ------

// Streaming (nontemporal) accesses for state that is touched once per step and
// is far larger than the caches; plain accesses otherwise.
typedef float nt_f4 __attribute__((ext_vector_type(4)));

template <bool NTL>
__device__ __forceinline__ float4 ld4(const float4 *p)
{
    if constexpr (NTL) {
        const nt_f4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_f4 *>(p));
        return make_float4(t.x, t.y, t.z, t.w);
    } else {
        return *p;
    }
}

template <bool NTL>
__device__ __forceinline__ void st4(float4 *p, const float4 v)
{
    if constexpr (NTL) {
        const nt_f4 t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<nt_f4 *>(p));
    } else {
        *p = v;
    }
}

__device__ __forceinline__ double dot4(const float4 a, const float4 b)
{
    double s = (double)a.x * (double)b.x;
    s = fma((double)a.y, (double)b.y, s);
    s = fma((double)a.z, (double)b.z, s);
    s = fma((double)a.w, (double)b.w, s);
    return s;
}

// Reduce N per-lane partial sums over aligned groups of W lanes.  Each halving
// step exchanges half of the remaining values with a partner lane of the other
// half; lanes keep the lower or upper half by their lane bit.  Returns, in every
// lane, the group total of value index (lane % W) / (W / N).
template <int W, int N>
__device__ __forceinline__ double head_reduce(const double *v, int lane)
{
    if constexpr (N == 1) {
        return group_sum<W>(v[0]);
    } else {
        constexpr int off = W / 2;
        const bool hi = (lane & off) != 0;
        double nv[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            if constexpr (off >= 16) {
                nv[i] = swap_sum<off>(v[i], v[N / 2 + i]);
            } else {
                const double mine = hi ? v[N / 2 + i] : v[i];
                const double send = hi ? v[i] : v[N / 2 + i];
                nv[i] = mine + partner<off>(send);
            }
        }
        return head_reduce<W / 2, N / 2>(nv, lane);
    }
}

}  // namespace o1
