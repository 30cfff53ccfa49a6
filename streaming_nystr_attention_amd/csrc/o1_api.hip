// Host side of the C ABI declared in include/o1.h: argument validation, state
// allocation (once, at o1_create_groups), stream-ordered launches, and field
// copies for tests.  No entry point synchronises with the host, except that a
// prefill needing a larger work buffer than it holds waits for its stream
// before freeing the old one, and o1_create_groups waits for the clearing of
// its new state's held value rows.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "o1.h"
#include "o1_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return O1_OK;
}

}  // namespace

struct o1_groups {
    o1_config cfg;
    int device;
    int G, R;
    int T;      // prompt length shared by every sealed layer
    int exact;  // that prompt took the exact-only mode
    std::vector<uint8_t> layer_sealed;
    std::vector<int64_t> layer_steps;  // decode steps since each layer's prefill
    o1::DevState st;                   // m_eff and pointers
    double *a64;                       // prefill work buffer: every head's exp-Gram
    size_t a64_bytes;
    size_t state_bytes;
    // exact-only mode: keys [G][exact_cap][d], values [G][exact_cap][dv], and the
    // split partials of its decode step (all allocated at create when exact_cap > 0)
    float *exact_k, *exact_v;
    double *exact_ws;
    size_t exact_ws_bytes;
    int32_t *exact_held;  // keys held per group [G], kept on the device
    double ridge_rel;     // relative ridge of the pinv (the page's RIDGE_REL unless set)
    size_t fold_bytes, ring_logit_bytes;  // parts of state_bytes (o1_info)
    // host copy of every head's ridge record, refreshed by o1_get_info after a
    // prefill or a write of the record (a diagnostics read, not on the hot path)
    mutable bool ridge_stale = true;
    mutable std::vector<double> lambda_host;
    mutable std::vector<int32_t> tries_host;

    bool any_sealed() const
    {
        return std::any_of(layer_sealed.begin(), layer_sealed.end(), [](uint8_t v) { return v != 0; });
    }
    bool all_sealed() const
    {
        return std::all_of(layer_sealed.begin(), layer_sealed.end(), [](uint8_t v) { return v != 0; });
    }
    // fewest / most decode steps over the sealed layers (0 when none is sealed)
    int64_t steps_extreme(bool largest) const
    {
        int64_t r = -1;
        for (size_t l = 0; l < layer_sealed.size(); ++l)
            if (layer_sealed[l] && (r < 0 || (largest ? layer_steps[l] > r : layer_steps[l] < r)))
                r = layer_steps[l];
        return r < 0 ? 0 : r;
    }
};

namespace {

// All groups of the handle (call index = group index).
o1::GroupMap whole_map(const o1_groups *g)
{
    return {g->G, g->cfg.n_kv, g->cfg.n_kv, 0};
}

// Layer l of every sequence: call index i = s * n_kv + kv.
o1::GroupMap layer_map(const o1_groups *g, int l)
{
    const o1_config &c = g->cfg;
    return {c.n_seq * c.n_kv, c.n_kv, c.n_layer * c.n_kv, l * c.n_kv};
}

struct FieldInfo {
    void *ptr;
    size_t bytes;
};

FieldInfo field_info(const o1_groups *g, int32_t field)
{
    const o1::DevState &s = g->st;
    const size_t G = (size_t)g->G, H = (size_t)s.hpk, m = (size_t)s.m;
    switch (field) {
    case O1_FIELD_NEAR_K: return {s.near_k, G * g->R * s.d * sizeof(float)};
    case O1_FIELD_NEAR_V: return {s.near_v, G * g->R * s.dv * sizeof(float)};
    case O1_FIELD_K_TILDE: return {s.k_tilde, G * m * s.d * sizeof(float)};
    case O1_FIELD_Q_TILDE: return {s.q_tilde, G * H * m * s.d * sizeof(float)};
    case O1_FIELD_MU: return {s.mu, G * H * m * m * sizeof(float)};
    case O1_FIELD_T_HAT: return {s.t_hat, G * H * m * s.dv * sizeof(float)};
    case O1_FIELD_Z_HAT: return {s.z_hat, G * H * m * sizeof(double)};
    case O1_FIELD_M_MAX: return {s.m_max, G * H * m * sizeof(float)};
    case O1_FIELD_WIN_HEAD: return {s.win_head, G * sizeof(int32_t)};
    case O1_FIELD_FAR_LEN: return {s.far_len, G * H * sizeof(int64_t)};
    case O1_FIELD_LAMBDA: return {s.lambda, G * H * sizeof(double)};
    case O1_FIELD_TRIES: return {s.tries, G * H * sizeof(int32_t)};
    case O1_FIELD_EXACT_K: return {g->exact_k, G * g->cfg.exact_cap * s.d * sizeof(float)};
    case O1_FIELD_EXACT_V: return {g->exact_v, G * g->cfg.exact_cap * s.dv * sizeof(float)};
    default: return {nullptr, 0};
    }
}

bool landmark_shaped(int32_t field)
{
    return field == O1_FIELD_K_TILDE || field == O1_FIELD_Q_TILDE || field == O1_FIELD_MU ||
           field == O1_FIELD_T_HAT || field == O1_FIELD_Z_HAT || field == O1_FIELD_M_MAX;
}

void free_state(o1_groups *g)
{
    o1::DevState &s = g->st;
    void *ptrs[] = {s.near_k, s.near_v,   s.k_tilde,  s.q_tilde,  s.mu,       s.t_hat,
                    s.z_hat,  s.m_max,    s.win_head, s.far_len,  s.lambda,   s.tries,
                    s.pend_v, s.pend_l,   s.m_ref,    s.ring_l,   g->a64,     g->exact_k,
                    g->exact_v, g->exact_ws, g->exact_held};
    for (void *p : ptrs)
        if (p) (void)hipFree(p);
}

// Makes the handle's device current for the scope of an entry point and
// restores the caller's device on exit.
class DeviceScope {
  public:
    explicit DeviceScope(const o1_groups *g)
    {
        if (hipGetDevice(&prev_) != hipSuccess) {
            rc_ = fail(O1_EHIP, "hipGetDevice failed");
        } else if (prev_ != g->device) {
            if (hipSetDevice(g->device) != hipSuccess)
                rc_ = fail(O1_EHIP, "hipSetDevice(%d) failed", g->device);
            else
                switched_ = true;
        }
    }
    ~DeviceScope()
    {
        if (switched_) (void)hipSetDevice(prev_);
    }
    int status() const { return rc_; }

  private:
    int prev_ = -1, rc_ = O1_OK;
    bool switched_ = false;
};

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

bool stride_ok(int64_t s) { return s >= 0 && s % 4 == 0; }

// Split partials of an exact-only step over `count` call indices, in doubles.
size_t exact_ws_doubles(int count, int hpk, int dv, int n_keys)
{
    const int splits = o1::exact_splits(count, n_keys);
    return splits == 1 ? 0 : (size_t)count * splits * hpk * (dv + 2);
}

// The prefill shared by o1_prefill (layer < 0: every group) and o1_prefill_layer.
int prefill_groups(o1_groups *g, int layer, const o1::PromptView &pv, int32_t T,
                   const o1_frozen *frozen, void *stream)
{
    const o1_config &c = g->cfg;
    const o1::GroupMap map = layer < 0 ? whole_map(g) : layer_map(g, layer);
    const bool exact = (long long)T <= (long long)c.w + c.sink + o1::kExactSlack;
    if (exact) {
        // exact-only mode (NystromGroup::prefill_shared): every key stays exact
        if (c.exact_cap == 0)
            return fail(O1_EEXACT,
                        "prompt of %d tokens is in the exact-only mode (T <= w + sink + %d = %d) "
                        "and the handle was created with exact_cap = 0",
                        T, o1::kExactSlack, c.w + c.sink + o1::kExactSlack);
        if (T > c.exact_cap)
            return fail(O1_EFULL, "exact-only prompt of %d tokens exceeds exact_cap = %d", T, c.exact_cap);
    } else if (!pv.q) {
        return fail(O1_EINVAL, "prefill: null queries");
    }
    if ((long long)T * map.count * c.hpk * c.d > (1LL << 40))
        return fail(O1_EINVAL, "prompt too large (T=%d)", T);
    DeviceScope dev(g);
    if (int rc = dev.status()) return rc;
    int m_eff = T / 8;
    if (m_eff < 4) m_eff = 4;
    if (m_eff > c.m) m_eff = c.m;

    if (!exact) {
        const size_t mp = (size_t)(m_eff + 15) / 16 * 16;  // zero-padded to whole 16 x 16 blocks
        const size_t need = sizeof(double) * (size_t)map.count * c.hpk * mp * mp;
        if (need > g->a64_bytes) {
            if (g->a64) {
                if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
                    return fail(O1_EHIP, "hipStreamSynchronize failed");
                (void)hipFree(g->a64);
                g->a64 = nullptr;
                g->a64_bytes = 0;
            }
            if (hipMalloc((void **)&g->a64, need) != hipSuccess) {
                (void)hipGetLastError();
                g->a64 = nullptr;
                return fail(O1_ENOMEM, "hipMalloc of %zu bytes of prefill work space failed", need);
            }
            g->a64_bytes = need;
        }
    }

    // A whole-handle prefill, or a layer prefill of another prompt length,
    // starts a new prompt: every layer is unsealed until sealed again (the
    // landmark count, hence the state layout, follows the prompt length).
    if (layer < 0 || !g->any_sealed() || T != g->T)
        std::fill(g->layer_sealed.begin(), g->layer_sealed.end(), 0);
    if (layer >= 0) g->layer_sealed[layer] = 0;
    g->T = T;
    g->exact = exact;
    g->st.m = exact ? 0 : m_eff;

    hipError_t err;
    if (exact) {
        err = o1::launch_exact_seal(g->st, pv, map, T, g->exact_k, g->exact_v, c.exact_cap,
                                    g->exact_held, (hipStream_t)stream);
    } else {
        o1::PrefillIO io;
        io.p = pv;
        io.map = map;
        io.T = T;
        io.fz_kt = frozen ? frozen->k_tilde : nullptr;
        io.fz_qt = frozen ? frozen->q_tilde : nullptr;
        io.fz_mu = frozen ? frozen->mu : nullptr;
        io.a64 = g->a64;
        io.ridge_rel = g->ridge_rel;
        err = o1::launch_prefill(g->st, io, (hipStream_t)stream);
    }
    g->ridge_stale = true;
    if (err != hipSuccess) return fail(O1_EHIP, "prefill launch failed: %s", hipGetErrorString(err));
    for (int l = 0; l < c.n_layer; ++l) {
        if (layer >= 0 && l != layer) continue;
        g->layer_sealed[l] = 1;
        g->layer_steps[l] = 0;
    }
    return ok();
}

// The decode step shared by o1_step (layer < 0: every group) and o1_step_layer.
int step_groups(o1_groups *g, int layer, const float *q, const float *k, const float *v, float *out,
                void *stream)
{
    if (!q || !k || !v || !out) return fail(O1_EINVAL, "step: null tensor");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(O1_EINVAL, "step: tensors must be 16-byte aligned");
    if (layer < 0 && !g->all_sealed())
        return fail(O1_ESTATE, "o1_step before every layer has a successful prefill");
    if (layer >= 0 && !g->layer_sealed[layer])
        return fail(O1_ESTATE, "o1_step_layer before a successful prefill of layer %d", layer);
    const o1::GroupMap map = layer < 0 ? whole_map(g) : layer_map(g, layer);
    hipError_t err;
    if (g->exact) {
        // Each group's key count is read on the device (and advanced there), so
        // layers stepped one by one may hold different counts and a captured
        // step replays correctly; the host mirror serves the checks below.
        const long long held =
            (long long)g->T + (layer < 0 ? g->steps_extreme(true) : g->layer_steps[layer]);
        if (held >= g->cfg.exact_cap)
            return fail(O1_EFULL, "exact-only groups already hold exact_cap = %d keys", g->cfg.exact_cap);
        DeviceScope dev(g);
        if (int rc = dev.status()) return rc;
        const int n = (int)held + 1;  // the fullest group's keys after this step's append
        o1::ExactIO io{};
        io.q = q;
        io.k = g->exact_k;
        io.v = g->exact_v;
        io.out = out;
        io.map = map;
        io.hpk = g->cfg.hpk;
        io.d = g->cfg.d;
        io.dv = g->cfg.dv;
        io.cap = g->cfg.exact_cap;
        io.first = 0;
        io.n_keys = n;
        int splits = o1::exact_splits(map.count, n);
        io.per_split = (n + splits - 1) / splits;
        splits = (n + io.per_split - 1) / io.per_split;
        io.scale = g->st.scale;
        const size_t parts = (size_t)map.count * splits * g->cfg.hpk;
        if (splits > 1) {
            io.ws_max = g->exact_ws;
            io.ws_sum = g->exact_ws + parts;
            io.ws_num = g->exact_ws + 2 * parts;
        }
        io.k_new = k;
        io.v_new = v;
        io.k_dst = g->exact_k;
        io.v_dst = g->exact_v;
        io.held = g->exact_held;
        err = o1::launch_exact(io, splits, (hipStream_t)stream);
    } else {
        DeviceScope dev(g);
        if (int rc = dev.status()) return rc;
        o1::DecodeIO io{q, k, v, out, map};
        err = o1::launch_decode(g->st, io, (hipStream_t)stream);
    }
    if (err != hipSuccess) return fail(O1_EHIP, "decode launch failed: %s", hipGetErrorString(err));
    for (int l = 0; l < g->cfg.n_layer; ++l)
        if (layer < 0 || l == layer) g->layer_steps[l] += 1;
    return ok();
}

}  // namespace

extern "C" {

int o1_abi_version(void) { return O1_ABI_VERSION; }

const char *o1_last_error(void) { return g_last_error.c_str(); }

int o1_create_groups(const o1_config *cfg, o1_groups **out)
{
    if (!cfg || !out) return fail(O1_EINVAL, "o1_create_groups: null argument");
    *out = nullptr;
    const o1_config c = *cfg;
    if (c.n_seq < 1 || c.n_layer < 1 || c.n_kv < 1)
        return fail(O1_EINVAL, "group counts must be >= 1 (n_seq=%d n_layer=%d n_kv=%d)", c.n_seq,
                    c.n_layer, c.n_kv);
    if (c.m < 4) return fail(O1_EINVAL, "landmark budget must be at least 4 (m=%d)", c.m);
    if (c.w < 1) return fail(O1_EINVAL, "window must hold at least one key (w=%d)", c.w);
    if (c.hpk < 1) return fail(O1_EINVAL, "a GQA group needs at least one query head (hpk=%d)", c.hpk);
    if (c.sink < 0) return fail(O1_EINVAL, "sink must be >= 0 (sink=%d)", c.sink);
    if (c.d < 1 || c.dv < 1) return fail(O1_EINVAL, "d and dv must be >= 1 (d=%d dv=%d)", c.d, c.dv);
    if (c.rect != O1_RECT_AGGREGATE && c.rect != O1_RECT_FM)
        return fail(O1_EINVAL, "unknown rectifier %d", c.rect);
    if (!(c.ridge_rel >= 0.0) || !isfinite(c.ridge_rel))
        return fail(O1_EINVAL, "ridge_rel must be finite and >= 0 (0 selects 1e-6), got %g", c.ridge_rel);
    const long long G = (long long)c.n_seq * c.n_layer * c.n_kv;
    if (G > (1LL << 30)) return fail(O1_EINVAL, "too many groups (%lld)", G);
    if (c.exact_cap < 0 || (double)G * c.exact_cap * ((double)c.d + c.dv) * 4.0 > 0x1p50)
        return fail(O1_EINVAL, "exact_cap must be >= 0 and its buffers below 2^50 bytes (exact_cap=%d)",
                    c.exact_cap);
    const int R = c.sink + c.w;
    const int m_cap = c.m < o1::kMaxLandmarks ? c.m : o1::kMaxLandmarks;
    if (!o1::decode_supported(c.d, c.dv, c.hpk, m_cap, R) || c.m > o1::kMaxLandmarks)
        return fail(O1_EUNSUPPORTED,
                    "shape not compiled: needs d == dv in {64,80,96,128,256} or d = 192 with dv = 128, hpk <= %d, "
                    "m <= %d, sink + w "
                    "<= 4096 with hpk'*(sink+w) <= 4096, hpk' = min(hpk, 8 (4 at d = 80)) rounded up to a power of two "
                    "(got d=%d dv=%d hpk=%d m=%d sink+w=%d)",
                    o1::kMaxHeads, o1::kMaxLandmarks, c.d, c.dv, c.hpk, c.m, R);

    o1_groups *g = new o1_groups();
    memset(&g->st, 0, sizeof g->st);
    g->cfg = c;
    g->G = (int)G;
    g->R = R;
    g->T = 0;
    g->exact = 0;
    g->layer_sealed.assign(c.n_layer, 0);
    g->layer_steps.assign(c.n_layer, 0);
    g->a64 = nullptr;
    g->a64_bytes = 0;
    g->exact_k = g->exact_v = nullptr;
    g->exact_ws = nullptr;
    g->exact_ws_bytes = 0;
    g->exact_held = nullptr;
    g->ridge_rel = c.ridge_rel > 0.0 ? c.ridge_rel : o1::kRidgeRel;
    if (hipGetDevice(&g->device) != hipSuccess) {
        delete g;
        return fail(O1_EHIP, "hipGetDevice failed");
    }
    o1::DevState &s = g->st;
    s.G = (int)G;
    s.hpk = c.hpk;
    s.d = c.d;
    s.dv = c.dv;
    s.w = c.w;
    s.sink = c.sink;
    s.R = R;
    s.rect = c.rect;
    s.m = 0;
    s.scale = 1.0f / sqrtf((float)c.d);

    const size_t Gs = (size_t)G, H = (size_t)c.hpk, M = (size_t)m_cap, E = (size_t)c.exact_cap;
    // split partials of the largest exact-only step, whole handle or one layer
    const size_t ws_bytes =
        E ? sizeof(double) * std::max(exact_ws_doubles((int)G, c.hpk, c.dv, c.exact_cap),
                                      exact_ws_doubles(c.n_seq * c.n_kv, c.hpk, c.dv, c.exact_cap))
          : 0;
    g->exact_ws_bytes = ws_bytes;
    struct Alloc {
        void **p;
        size_t bytes;
    } allocs[] = {
        {(void **)&s.near_k, Gs * R * c.d * sizeof(float)},
        {(void **)&s.near_v, Gs * R * c.dv * sizeof(float)},
        {(void **)&s.k_tilde, Gs * M * c.d * sizeof(float)},
        {(void **)&s.q_tilde, Gs * H * M * c.d * sizeof(float)},
        {(void **)&s.mu, Gs * H * M * M * sizeof(float)},
        {(void **)&s.t_hat, Gs * H * M * c.dv * sizeof(float)},
        {(void **)&s.z_hat, Gs * H * M * sizeof(double)},
        {(void **)&s.m_max, Gs * H * M * sizeof(float)},
        {(void **)&s.win_head, Gs * sizeof(int32_t)},
        {(void **)&s.far_len, Gs * H * sizeof(int64_t)},
        {(void **)&s.lambda, Gs * H * sizeof(double)},
        {(void **)&s.tries, Gs * H * sizeof(int32_t)},
        {(void **)&s.pend_v, Gs * o1::kPend * c.dv * sizeof(float)},
        {(void **)&s.pend_l, Gs * H * o1::kPend * M * sizeof(double)},
        {(void **)&s.m_ref, Gs * H * M * sizeof(float)},
        {(void **)&s.ring_l, c.w >= o1::kPend ? Gs * c.w * H * M * sizeof(double) : 0},
        {(void **)&g->exact_k, Gs * E * c.d * sizeof(float)},
        {(void **)&g->exact_v, Gs * E * c.dv * sizeof(float)},
        {(void **)&g->exact_ws, ws_bytes},
        {(void **)&g->exact_held, E ? Gs * sizeof(int32_t) : 0},
    };
    size_t total = 0;
    for (auto &a : allocs) {
        if (a.bytes == 0) continue;  // exact-only buffers of a handle without that mode
        if (hipMalloc(a.p, a.bytes) != hipSuccess) {
            (void)hipGetLastError();
            free_state(g);
            delete g;
            return fail(O1_ENOMEM, "hipMalloc of %zu bytes failed", a.bytes);
        }
        total += a.bytes;
    }
    // held value rows start at zero: a slot the held count does not cover is
    // never read, and an empty covered slot (logits -inf) weighs 0, which must
    // not meet a non-finite row
    if (hipMemsetAsync(s.pend_v, 0, Gs * o1::kPend * c.dv * sizeof(float), nullptr) != hipSuccess ||
        hipStreamSynchronize(nullptr) != hipSuccess) {
        (void)hipGetLastError();
        free_state(g);
        delete g;
        return fail(O1_EHIP, "clearing the held value rows failed");
    }
    g->state_bytes = total;
    g->fold_bytes = Gs * o1::kPend * c.dv * sizeof(float) + Gs * H * o1::kPend * M * sizeof(double) +
                    Gs * H * M * sizeof(float);
    g->ring_logit_bytes = c.w >= o1::kPend ? Gs * c.w * H * M * sizeof(double) : 0;
    // the decode streams its state from HBM when the state outgrows the cache
    const size_t exact_bytes = Gs * E * (c.d + c.dv) * sizeof(float) + ws_bytes;
    s.stream_state = total - std::min(total, exact_bytes) > o1::kInfinityCacheBytes ? 1 : 0;
    *out = g;
    return ok();
}

void o1_destroy_groups(o1_groups *g)
{
    if (!g) return;
    DeviceScope dev(g);
    free_state(g);
    delete g;
}

int o1_prefill(o1_groups *g, const float *q, const float *k, const float *v, int32_t T,
               const o1_frozen *frozen, void *stream)
{
    if (!g || !k || !v) return fail(O1_EINVAL, "o1_prefill: null argument");
    if (T < 1) return fail(O1_EINVAL, "prompt length must be >= 1 (T=%d)", T);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(O1_EINVAL, "o1_prefill: tensors must be 16-byte aligned");
    const o1_config &c = g->cfg;
    // q [G][hpk][T][d], k [G][T][d], v [G][T][dv], seen as call index i = group
    // = (s * n_layer + l) * n_kv + kv with outer index i / n_kv and KV head i % n_kv
    o1::PromptView pv;
    pv.q = q;
    pv.k = k;
    pv.v = v;
    pv.q_outer = (int64_t)c.n_kv * c.hpk * T * c.d;
    pv.q_head = (int64_t)T * c.d;
    pv.q_pos = c.d;
    pv.k_outer = (int64_t)c.n_kv * T * c.d;
    pv.k_inner = (int64_t)T * c.d;
    pv.k_pos = c.d;
    pv.v_outer = (int64_t)c.n_kv * T * c.dv;
    pv.v_inner = (int64_t)T * c.dv;
    pv.v_pos = c.dv;
    return prefill_groups(g, -1, pv, T, frozen, stream);
}

int o1_prefill_layer(o1_groups *g, int32_t layer, const o1_prompt_view *p, int32_t T,
                     const o1_frozen *frozen, void *stream)
{
    if (!g || !p || !p->k || !p->v) return fail(O1_EINVAL, "o1_prefill_layer: null argument");
    if (layer < 0 || layer >= g->cfg.n_layer)
        return fail(O1_EINVAL, "layer %d out of range (n_layer=%d)", layer, g->cfg.n_layer);
    if (T < 1) return fail(O1_EINVAL, "prompt length must be >= 1 (T=%d)", T);
    if (!aligned16(p->q) || !aligned16(p->k) || !aligned16(p->v))
        return fail(O1_EINVAL, "o1_prefill_layer: tensors must be 16-byte aligned");
    if (!stride_ok(p->q_seq) || !stride_ok(p->q_head) || !stride_ok(p->q_pos) || !stride_ok(p->k_seq) ||
        !stride_ok(p->k_kv) || !stride_ok(p->k_pos) || !stride_ok(p->v_seq) || !stride_ok(p->v_kv) ||
        !stride_ok(p->v_pos))
        return fail(O1_EINVAL, "o1_prefill_layer: strides must be non-negative multiples of 4 floats");
    o1::PromptView pv;
    pv.q = p->q;
    pv.k = p->k;
    pv.v = p->v;
    pv.q_outer = p->q_seq;
    pv.q_head = p->q_head;
    pv.q_pos = p->q_pos;
    pv.k_outer = p->k_seq;
    pv.k_inner = p->k_kv;
    pv.k_pos = p->k_pos;
    pv.v_outer = p->v_seq;
    pv.v_inner = p->v_kv;
    pv.v_pos = p->v_pos;
    return prefill_groups(g, layer, pv, T, frozen, stream);
}

int o1_step(o1_groups *g, const float *q, const float *k, const float *v, float *out, void *stream)
{
    if (!g) return fail(O1_EINVAL, "o1_step: null argument");
    return step_groups(g, -1, q, k, v, out, stream);
}

int o1_step_layer(o1_groups *g, int32_t layer, const float *q, const float *k, const float *v,
                  float *out, void *stream)
{
    if (!g) return fail(O1_EINVAL, "o1_step_layer: null argument");
    if (layer < 0 || layer >= g->cfg.n_layer)
        return fail(O1_EINVAL, "layer %d out of range (n_layer=%d)", layer, g->cfg.n_layer);
    return step_groups(g, layer, q, k, v, out, stream);
}

int o1_get_info(const o1_groups *g, o1_info *info)
{
    if (!g || !info) return fail(O1_EINVAL, "o1_get_info: null argument");
    const bool any = g->any_sealed();
    info->n_groups = g->G;
    info->sealed = g->all_sealed();
    info->prompt_len = any ? g->T : 0;
    info->m_eff = any ? g->st.m : 0;
    info->steps = g->steps_extreme(false);
    info->state_bytes = g->state_bytes;
    info->work_bytes = g->a64_bytes;
    info->exact_only = any ? g->exact : 0;
    info->exact_keys = !any ? 0 : g->exact ? (int32_t)(g->T + g->steps_extreme(true)) : g->R;
    info->n_layer = g->cfg.n_layer;
    info->layers_sealed = (int32_t)std::count(g->layer_sealed.begin(), g->layer_sealed.end(), 1);
    info->max_steps = g->steps_extreme(true);
    info->fold_bytes = g->fold_bytes;
    info->ring_logit_bytes = g->ring_logit_bytes;

    // NystromState::memory_bytes (f32 words by vector length) of every sealed group
    const o1_config &c = g->cfg;
    const uint64_t per_layer = (uint64_t)c.n_seq * c.n_kv, d = c.d, dv = c.dv, H = c.hpk;
    uint64_t words = 0;
    for (int l = 0; l < c.n_layer; ++l) {
        if (!g->layer_sealed[l]) continue;
        uint64_t w_group;
        if (g->exact) {
            const uint64_t n = (uint64_t)g->T + (uint64_t)g->layer_steps[l];
            w_group = n * (d + dv) + (g->layer_steps[l] > 0 ? H * n : 0);
        } else {
            const uint64_t m = (uint64_t)g->st.m, S = c.sink, W = c.w;
            w_group = W * (d + dv) + S * (d + dv) + m * d +
                      H * (m * dv + m + m + m * d + m * m + (S + W) + 3 * m);
        }
        words += per_layer * w_group;
    }
    info->page_bytes = words * sizeof(float);

    // ridge record of the sealed skeleton layers' computed pinvs
    info->lambda_min = info->lambda_median = info->lambda_max = 0.0;
    info->tries_max = info->heads_retried = info->heads_fallback = info->ridge_heads = 0;
    if (any && !g->exact) {
        const size_t n = (size_t)g->G * c.hpk;
        if (g->ridge_stale) {
            DeviceScope dev(g);
            if (int rc = dev.status()) return rc;
            g->lambda_host.resize(n);
            g->tries_host.resize(n);
            if (hipDeviceSynchronize() != hipSuccess ||
                hipMemcpy(g->lambda_host.data(), g->st.lambda, n * sizeof(double), hipMemcpyDeviceToHost) !=
                    hipSuccess ||
                hipMemcpy(g->tries_host.data(), g->st.tries, n * sizeof(int32_t), hipMemcpyDeviceToHost) !=
                    hipSuccess) {
                (void)hipGetLastError();
                return fail(O1_EHIP, "o1_get_info: reading the ridge record failed");
            }
            g->ridge_stale = false;
        }
        std::vector<double> lam;
        lam.reserve(n);
        for (size_t i = 0; i < n; ++i) {
            const int l = (int)((i / c.hpk / c.n_kv) % c.n_layer);
            const int32_t t = g->tries_host[i];
            if (!g->layer_sealed[l] || t < 1) continue;  // unsealed layer, or M given frozen
            lam.push_back(g->lambda_host[i]);
            info->tries_max = std::max(info->tries_max, t);
            info->heads_retried += t > 1;
            info->heads_fallback += t > o1::kRidgeTries;
        }
        if (!lam.empty()) {
            std::sort(lam.begin(), lam.end());
            const size_t k = lam.size();
            info->lambda_min = lam.front();
            info->lambda_max = lam.back();
            info->lambda_median = k % 2 ? lam[k / 2] : 0.5 * (lam[k / 2 - 1] + lam[k / 2]);
            info->ridge_heads = (int32_t)k;
        }
    }
    return ok();
}

int o1_field_bytes(const o1_groups *g, int32_t field, size_t *bytes)
{
    if (!g || !bytes) return fail(O1_EINVAL, "o1_field_bytes: null argument");
    if (field < 0 || field >= O1_FIELD_COUNT) return fail(O1_EINVAL, "unknown field %d", field);
    if ((field == O1_FIELD_EXACT_K || field == O1_FIELD_EXACT_V) && g->cfg.exact_cap == 0)
        return fail(O1_EINVAL, "field %d: the handle was created with exact_cap = 0", field);
    if (landmark_shaped(field) && (!g->any_sealed() || g->exact))
        return fail(O1_ESTATE, "field %d has no shape before a skeleton-mode prefill", field);
    *bytes = field_info(g, field).bytes;
    return ok();
}

int o1_read_field(const o1_groups *g, int32_t field, void *dst, size_t bytes, void *stream)
{
    size_t want = 0;
    int rc = o1_field_bytes(g, field, &want);
    if (rc) return rc;
    if (!dst) return fail(O1_EINVAL, "o1_read_field: null destination");
    if (bytes != want) return fail(O1_EINVAL, "field %d holds %zu bytes, not %zu", field, want, bytes);
    DeviceScope dev(g);
    if ((rc = dev.status())) return rc;
    const hipStream_t st = (hipStream_t)stream;
    if (field == O1_FIELD_T_HAT) {
        // T^ with the held evictions folded in, built in a stream-ordered
        // temporary; the state itself is left as it is
        void *tmp = nullptr;
        hipError_t err = hipMallocAsync(&tmp, bytes, st);
        if (err != hipSuccess) {
            (void)hipGetLastError();
            return fail(O1_ENOMEM, "hipMallocAsync of %zu bytes failed: %s", bytes, hipGetErrorString(err));
        }
        err = o1::launch_fold(g->st, static_cast<float *>(tmp), false, st);
        if (err == hipSuccess) err = hipMemcpyAsync(dst, tmp, bytes, hipMemcpyDefault, st);
        const hipError_t ferr = hipFreeAsync(tmp, st);
        if (err == hipSuccess) err = ferr;
        if (err != hipSuccess) return fail(O1_EHIP, "reading T^ failed: %s", hipGetErrorString(err));
        return ok();
    }
    hipError_t err = hipMemcpyAsync(dst, field_info(g, field).ptr, bytes, hipMemcpyDefault, st);
    if (err != hipSuccess) return fail(O1_EHIP, "hipMemcpyAsync failed: %s", hipGetErrorString(err));
    return ok();
}

int o1_write_field(o1_groups *g, int32_t field, const void *src, size_t bytes, void *stream)
{
    if (g && !g->any_sealed()) return fail(O1_ESTATE, "o1_write_field before a successful prefill");
    size_t want = 0;
    int rc = o1_field_bytes(g, field, &want);
    if (rc) return rc;
    if (!src) return fail(O1_EINVAL, "o1_write_field: null source");
    if (bytes != want) return fail(O1_EINVAL, "field %d holds %zu bytes, not %zu", field, want, bytes);
    DeviceScope dev(g);
    if ((rc = dev.status())) return rc;
    const hipStream_t st = (hipStream_t)stream;
    o1::DevState &s = g->st;
    hipError_t err = hipSuccess;
    // fold the held evictions into T^ first, so that what is written meets a
    // state with none held (T^ at scale e^{-m_max})
    if (s.m > 0) err = o1::launch_fold(s, s.t_hat, true, st);
    if (err == hipSuccess) err = hipMemcpyAsync(field_info(g, field).ptr, src, bytes, hipMemcpyDefault, st);
    // T^ is stored at the scale of the running max it was written against
    if (err == hipSuccess && field == O1_FIELD_M_MAX)
        err = hipMemcpyAsync(s.m_ref, s.m_max, bytes, hipMemcpyDeviceToDevice, st);
    // the far-insert logits kept per ring slot: recomputed for every key in the
    // ring, since a write may change the ring's keys or q~, or far_len / win_head,
    // which schedule the folds that compute the logits of newly arrived keys
    if (err == hipSuccess && s.m > 0) err = o1::launch_ring_logits(s, whole_map(g), st);
    if (field == O1_FIELD_LAMBDA || field == O1_FIELD_TRIES) g->ridge_stale = true;
    if (err != hipSuccess) return fail(O1_EHIP, "writing field %d failed: %s", field, hipGetErrorString(err));
    return ok();
}

}  // extern "C"

// ---- the work space of o1_exact_attend_noalloc ---------------------------
// One array per device, in the code object's device memory: the split
// partials (max, sum, numerator) of a launch.  In host code `scratch` names a
// host-side shadow, not device memory: its device address is looked up with
// hipGetSymbolAddress, per device, on that device's first call, and only that
// address is passed to kernels.  Every partial a launch reads it has written
// in the same launch, so nothing needs clearing between calls.
namespace {
constexpr size_t kScratchBytes = O1_EXACT_NOALLOC_BYTES;
constexpr int kMaxDevices = 64;
}  // namespace
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

namespace {
std::mutex g_scratch_mu;
double *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, null until looked up

int scratch_of_current_device(double **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(O1_EHIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(O1_EUNSUPPORTED, "o1_exact_attend_noalloc: device %d beyond the %d supported", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(O1_EHIP, "hipGetSymbolAddress of the static work space failed on device %d: %s",
                        dev, hipGetErrorString(err));
        }
        g_scratch_ptr[dev] = static_cast<double *>(p);
    }
    *out = g_scratch_ptr[dev];
    return O1_OK;
}
}  // namespace

extern "C" {

static int exact_check(const o1_exact_desc *x, int *splits, size_t *bytes)
{
    if (!x) return fail(O1_EINVAL, "o1_exact: null descriptor");
    if (x->n_groups < 1 || x->hpk < 1 || x->d < 1 || x->dv < 1 || x->cap < 1)
        return fail(O1_EINVAL, "o1_exact: sizes must be >= 1");
    if (x->n_keys < 1 || x->n_keys > x->cap || x->first < 0 || x->first >= x->n_keys)
        return fail(O1_EINVAL, "o1_exact: need 0 <= first < n_keys <= cap (first=%d n_keys=%d cap=%d)",
                    x->first, x->n_keys, x->cap);
    if (!o1::widths_compiled(x->d, x->dv) || x->hpk > o1::kMaxHeads)
        return fail(O1_EUNSUPPORTED,
                    "o1_exact: compiled for d == dv in {64,80,96,128,256} or d = 192 with dv = 128, hpk <= %d",
                    o1::kMaxHeads);
    *splits = o1::exact_splits(x->n_groups, x->n_keys - x->first);
    *bytes = *splits == 1 ? 0
                          : sizeof(double) * (size_t)x->n_groups * *splits * x->hpk * (x->dv + 2);
    return O1_OK;
}

int o1_exact_workspace_bytes(const o1_exact_desc *desc, size_t *bytes)
{
    if (!bytes) return fail(O1_EINVAL, "o1_exact_workspace_bytes: null argument");
    int splits = 0;
    int rc = exact_check(desc, &splits, bytes);
    return rc ? rc : ok();
}

// The launch shared by o1_exact_attend and o1_exact_attend_noalloc, after
// their checks: `ws` holds the split partials (null when splits == 1).
static int exact_launch(const o1_exact_desc &x, int splits, const float *q, const float *k,
                        const float *v, float *out, double *ws, void *stream)
{
    o1::ExactIO io{};
    io.q = q;
    io.k = k;
    io.v = v;
    io.out = out;
    io.map = {x.n_groups, x.n_groups, 0, 0};  // cache group = call index
    io.hpk = x.hpk;
    io.d = x.d;
    io.dv = x.dv;
    io.cap = x.cap;
    io.first = x.first;
    io.n_keys = x.n_keys;
    const int visible = x.n_keys - x.first;
    io.per_split = (visible + splits - 1) / splits;
    splits = (visible + io.per_split - 1) / io.per_split;  // no empty ranges
    io.scale = x.scale > 0.0f ? x.scale : 1.0f / sqrtf((float)x.d);
    const size_t parts = (size_t)x.n_groups * splits * x.hpk;
    io.ws_max = ws;
    io.ws_sum = ws ? ws + parts : nullptr;
    io.ws_num = ws ? ws + 2 * parts : nullptr;
    hipError_t err = o1::launch_exact(io, splits, (hipStream_t)stream);
    if (err != hipSuccess) return fail(O1_EHIP, "exact attention launch failed: %s", hipGetErrorString(err));
    return ok();
}

static int exact_tensors_check(const char *who, const float *q, const float *k, const float *v,
                               const float *out)
{
    if (!q || !k || !v || !out) return fail(O1_EINVAL, "%s: null tensor", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(O1_EINVAL, "%s: tensors must be 16-byte aligned", who);
    return O1_OK;
}

int o1_exact_attend(const o1_exact_desc *desc, const float *q, const float *k, const float *v,
                    float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    int splits = 0;
    size_t need = 0;
    int rc = exact_check(desc, &splits, &need);
    if (rc) return rc;
    if ((rc = exact_tensors_check("o1_exact_attend", q, k, v, out))) return rc;
    if (need && (!workspace || workspace_bytes < need))
        return fail(O1_EINVAL, "o1_exact_attend: work space of %zu bytes needed", need);
    return exact_launch(*desc, splits, q, k, v, out, static_cast<double *>(workspace), stream);
}

int o1_exact_attend_noalloc(const o1_exact_desc *desc, const float *q, const float *k, const float *v,
                            float *out, void *stream)
{
    int splits = 0;
    size_t need = 0;
    int rc = exact_check(desc, &splits, &need);
    if (rc) return rc;
    if ((rc = exact_tensors_check("o1_exact_attend_noalloc", q, k, v, out))) return rc;
    if (need > kScratchBytes)
        return fail(O1_EINVAL,
                    "o1_exact_attend_noalloc: this launch needs %zu bytes of work space, more than the "
                    "%zu bytes of its static buffer (o1_exact_attend takes a caller work space)",
                    need, kScratchBytes);
    double *ws = nullptr;
    if (need && (rc = scratch_of_current_device(&ws))) return rc;
    return exact_launch(*desc, splits, q, k, v, out, ws, stream);
}

}  // extern "C"
