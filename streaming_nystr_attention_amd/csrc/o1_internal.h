// Internal interface between the C-ABI host code (o1_api.hip) and the gfx950
// kernels (o1_decode.hip, o1_prefill.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace o1 {

constexpr int kMaxLandmarks = 64;      // largest m_eff the kernels are compiled for
constexpr double kDenEps = 1e-30;      // DEN_EPS of the nystrom.rs source page
constexpr double kRidgeRel = 1e-6;     // RIDGE_REL of the nystrom.rs source page
constexpr int kRidgeTries = 12;        // ridge_pinv: attempts before the fallback
constexpr int kExactSlack = 8;         // EXACT_SLACK of the nystrom.rs source page

// Device state of G independent groups (one GQA group each).  Layout, with
// R = sink + w near rows and m = m_eff:
//   near_k [G][R][d], near_v [G][R][dv]   rows 0..sink-1 sinks, row sink+s ring slot s
//   k_tilde [G][m][d]                     key landmarks (f32)
//   q_tilde [G][hpk][m][d]                query landmarks (f32)
//   mu      [G][hpk][m][m]                mixing matrix, row = key landmark
//   t_hat   [G][hpk][m][dv] (f32), z_hat [G][hpk][m] (f64), m_max [G][hpk][m] (f32)
//   win_head [G] (i32), far_len [G][hpk] (i64), lambda [G][hpk] (f64), tries [G][hpk] (i32)
struct DevState {
    int G, hpk, d, dv, w, sink, R, rect;
    int m;        // m_eff of the current prefill
    float scale;  // f32 1/sqrt(d), as NystromGroup::prefill_shared sets it
    float *near_k, *near_v, *k_tilde, *q_tilde, *mu, *t_hat, *m_max;
    double *z_hat, *lambda;
    int32_t *win_head, *tries;
    int64_t *far_len;
};

struct DecodeIO {
    const float *q, *k, *v;
    float *out;
};

struct PrefillIO {
    const float *q, *k, *v;  // prompt [G][hpk][T][d], [G][T][d], [G][T][dv]
    int T;
    const float *fz_kt, *fz_qt, *fz_mu;  // optional frozen replacements
    double *lm64;                        // work: [G][1 + hpk][m][d] f64 landmarks
};

// True when the decode kernel is compiled for this shape.
bool decode_supported(int d, int dv, int hpk, int m, int R);
hipError_t launch_decode(const DevState &s, const DecodeIO &io, hipStream_t stream);
hipError_t launch_prefill(const DevState &s, const PrefillIO &io, hipStream_t stream);

// ---- wavefront helpers (wave64) ------------------------------------------

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of
// the group receives the group total.
template <int W>
__device__ __forceinline__ double group_sum(double x)
{
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__device__ __forceinline__ double wave_sum(double x) { return group_sum<64>(x); }

__device__ __forceinline__ double wave_max(double x)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmax(x, __shfl_xor(x, off, 64));
    return x;
}

}  // namespace o1
