// Prefill freeze of streaming Nystrom attention for every group at once:
// NystromGroup::prefill_shared, NystromHead::seal, ridge_pinv / cholesky and
// the replay of NystromState::prefill_group on the nystrom.rs source page.
//
//   landmarks_kernel   grid G: segment means of the keys (K~) and then of each
//                      head's queries (Q~), f64 accumulation in row order, stored
//                      f32 (state) and kept f64 in LDS for the exp-Gram A =
//                      exp(Q~ K~^T * scale) (f64 MFMA), written per head to the
//                      work buffer; the key rows of the sinks and the ring are
//                      copied to the state as the key pass streams them.
//   scatter_kernel     grid G: the value rows of the sinks (prompt rows
//                      0..sink-1) and the ring (the last w prompt rows, row j in
//                      slot (j - sink) mod w) -- the key rows too when frozen key
//                      landmarks skip the key pass --, the ring head and
//                      far_len after the replay, and an empty set of evictions
//                      held apart from T^ (logits -inf).
//   gram_pinv_kernel   grid G * hpk: G = A^T A on f64 MFMA from the exp-Gram,
//                      lambda = ridge_rel * max(mean diag G, DBL_MIN), Cholesky of
//                      G + lambda I in LDS (lambda x10 on a failed pivot, up to 12
//                      attempts, then diag(1/mean diag)), M = (G + lambda I)^-1 A^T
//                      by substitutions spread over lane groups.  Two m x m f64
//                      matrices of LDS per head.
//   far_mfma_kernel    grid G * ceil(hpk / HB): the far field of keys sink .. T-w-1, i.e. the
//                      state the page's sequential replay through far_insert
//                      reaches, computed in 16-key tiles on f64 MFMA with an
//                      online per-landmark max: m_max_i = max_j l_ij,
//                      Z^_i = sum_j e^{l_ij - m_max_i}, T^_i = sum_j e^{l_ij - m_max_i} v_j.
//
// G above is the number of groups a launch covers, given by a GroupMap (the
// whole handle, or one layer of every sequence): the prompt is read in place
// through a PromptView by the launch's own index, the state is written at the
// mapped group.
#include <float.h>

#include "o1_internal.h"

namespace o1 {
namespace {

constexpr int kThreads = 256;

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kLmThreads = 512;

// Near-state row of prompt key j, or -1: sinks j < sink keep row j, the last w
// keys go to ring slot (j - sink) mod w (row sink + slot).
__device__ __forceinline__ int near_row(int j, int S, int w, int T)
{
    if (j < S) return j;
    if (j >= T - w) return S + (j - S) % w;
    return -1;
}

// Segment means of the rows of x (row stride pos floats) into dst32 (state, f32)
// and l64 (LDS, f64, row stride ld): one thread per (segment, 4 components),
// the segment's rows summed in row order, eight rows' loads in flight at a
// time.  With `near`, rows that are sinks or ring keys are also copied there.
__device__ __forceinline__ void seg_means_pass(const float *x, int64_t pos, int T, int m, int d,
                                               float *dst32, double *l64, int ld, float4 *near,
                                               int S, int w)
{
    const int d4 = d / 4;
    for (int t = threadIdx.x; t < m * d4; t += kLmThreads) {
        const int a = t / d4, c4 = t - a * d4, c = c4 * 4;
        const int lo = (int)((long)a * T / m), hi = (int)((long)(a + 1) * T / m);
        double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
        const float *col = x + c;
        // only the first and last segments can hold sinks or ring keys
        const bool copy = near && (lo < S || hi > T - w);
        int j = lo;
        for (; j + 8 <= hi; j += 8) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4 *>(col + (int64_t)(j + u) * pos);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s0 += (double)v[u].x;
                s1 += (double)v[u].y;
                s2 += (double)v[u].z;
                s3 += (double)v[u].w;
            }
            if (copy) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int r = near_row(j + u, S, w, T);
                    if (r >= 0) near[(size_t)r * d4 + c4] = v[u];
                }
            }
        }
        for (; j < hi; ++j) {
            const float4 v = *reinterpret_cast<const float4 *>(col + (int64_t)j * pos);
            s0 += (double)v.x;
            s1 += (double)v.y;
            s2 += (double)v.z;
            s3 += (double)v.w;
            if (copy) {
                const int r = near_row(j, S, w, T);
                if (r >= 0) near[(size_t)r * d4 + c4] = v;
            }
        }
        const double inv = 1.0 / (double)(hi - lo);
        const double mean[4] = {s0 * inv, s1 * inv, s2 * inv, s3 * inv};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            l64[a * ld + c + e] = mean[e];
            dst32[a * d + c + e] = (float)mean[e];
        }
    }
}

// Frozen landmarks given by the caller: the state takes them, LDS their f64 values.
__device__ __forceinline__ void frozen_pass(const float *fz, int m, int d, float *dst32, double *l64, int ld)
{
    for (int t = threadIdx.x; t < m * d; t += kLmThreads) {
        const int a = t / d, c = t - a * d;
        const float v = fz[t];
        dst32[t] = v;
        l64[a * ld + c] = (double)v;
    }
}

// One work-group per group, 512 threads (two per CU, as LDS allows at m <= 32,
// d = 128: four waves per SIMD); dynamic LDS: K~ and one head's Q~ in
// f64, [mp][d + 1] each (mp = m rounded up to 16, rows past m zero).  The
// exp-Gram of head h, A[i][j] = exp(q~_i . k~_j * scale), runs on
// v_mfma_f64_16x16x4f64 from LDS, one 16 x 16 block per wave, and goes to
// io.a64[call][h][m][m] for gram_pinv_kernel (`gram` = 0: M is given frozen and
// no A is needed).
__global__ __launch_bounds__(kLmThreads, 4) void landmarks_kernel(DevState s, PrefillIO io, int gram)
{
    const int ci = blockIdx.x, g = io.map.state(ci);
    const int d = s.d, m = s.m, T = io.T, H = s.hpk, tid = threadIdx.x;
    const int nb = (m + 15) / 16, mp = nb * 16, ld = d + 1;
    extern __shared__ double lm_lds[];
    double *kt64 = lm_lds, *qt64 = lm_lds + (size_t)mp * ld;
    // rows past m stay zero for every head
    for (int t = tid; t < (mp - m) * ld; t += kLmThreads) {
        kt64[m * ld + t] = 0.0;
        qt64[m * ld + t] = 0.0;
    }

    float *kt32 = s.k_tilde + (size_t)g * m * d;
    if (io.fz_kt) {
        frozen_pass(io.fz_kt + (size_t)ci * m * d, m, d, kt32, kt64, ld);
    } else {
        float4 *near = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * s.R * (d / 4);
        seg_means_pass(io.p.k_row(io.map, ci, 0), io.p.k_pos, T, m, d, kt32, kt64, ld, near, s.sink, s.w);
    }

    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    const double sc = (double)s.scale;
    for (int h = 0; h < H; ++h) {
        float *qt32 = s.q_tilde + ((size_t)g * H + h) * m * d;
        __syncthreads();  // the previous head's exp-Gram is done with qt64
        if (io.fz_qt)
            frozen_pass(io.fz_qt + ((size_t)ci * H + h) * m * d, m, d, qt32, qt64, ld);
        else
            seg_means_pass(io.p.q_row(io.map, H, ci, h, 0), io.p.q_pos, T, m, d, qt32, qt64, ld, nullptr,
                           0, 0);
        if (!gram) continue;
        __syncthreads();
        double *a = io.a64 + ((size_t)ci * H + h) * m * m;
        for (int blk = wave; blk < nb * nb; blk += kLmThreads / 64) {
            const int bi = blk / nb, bj = blk - bi * nb;
            const double *qrow = qt64 + (bi * 16 + li) * ld + lk;
            const double *krow = kt64 + (bj * 16 + li) * ld + lk;
            f64x4 acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
            // k-step ks covers components 4 ks .. 4 ks + 3 (k-lane lk: 4 ks + lk)
            for (int ks = 0; ks < d / 4; ks += 2) {
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qrow[4 * ks], krow[4 * ks], acc, 0, 0, 0);
                acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(qrow[4 * ks + 4], krow[4 * ks + 4], acc2, 0, 0, 0);
            }
            acc += acc2;
            // lane holds A[bi*16 + lk + 4 r][bj*16 + li]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = bi * 16 + lk + 4 * r, j = bj * 16 + li;
                if (i < m && j < m) a[i * m + j] = exp(acc[r] * sc);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(DevState s, PrefillIO io)
{
    const int ci = blockIdx.x, g = io.map.state(ci);
    const int S = s.sink, w = s.w, R = s.R, T = io.T;
    const int ck = s.d / 4, cv = s.dv / 4;
    const float4 *kin = reinterpret_cast<const float4 *>(io.p.k_row(io.map, ci, 0));
    const float4 *vin = reinterpret_cast<const float4 *>(io.p.v_row(io.map, ci, 0));
    const int64_t kp = io.p.k_pos / 4, vp = io.p.v_pos / 4;  // row strides in float4
    float4 *nk = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * R * ck;
    float4 *nv = reinterpret_cast<float4 *>(s.near_v) + (size_t)g * R * cv;
    const int base = T - w;          // first prompt key still in the window
    const int shift = base - S;      // >= 9 in skeleton mode
    // the key rows come from the landmark kernel's key pass unless frozen key
    // landmarks replaced it
    const int kc = io.fz_kt ? ck : 0;
    for (int t = threadIdx.x; t < R * (kc + cv); t += kThreads) {
        const int r = t / (kc + cv), c = t - r * (kc + cv);
        int j;
        if (r < S) {
            j = r;
        } else {
            const int slot = r - S;
            j = base + ((slot - shift) % w + w) % w;  // (j - S) mod w == slot
        }
        if (c < kc) nk[(size_t)r * ck + c] = kin[(int64_t)j * kp + c];
        else nv[(size_t)r * cv + (c - kc)] = vin[(int64_t)j * vp + (c - kc)];
    }
    const int evictions = T - S - w;
    if (threadIdx.x == 0) s.win_head[g] = evictions % w;
    for (int h = threadIdx.x; h < s.hpk; h += kThreads) s.far_len[(size_t)g * s.hpk + h] = evictions;
    // no evictions held apart from T^ yet: every slot's logits -inf (weight 0;
    // the value rows stay finite from the handle's creation or earlier use)
    double *pl = s.pend_l + (size_t)g * s.hpk * kPend * s.m;
    for (int t = threadIdx.x; t < s.hpk * kPend * s.m; t += kThreads) pl[t] = -__builtin_inf();
}

// One block per (group, head), 256 threads.  Dynamic LDS: A [mp][gram_lda(mp)]
// and L [mp][mp + 1], f64, with mp = m rounded up to 16 (padding rows/columns of
// A are 0).  A^T A runs on v_mfma_f64_16x16x4f64 (operand layout: A[i][k] in
// lane i + 16 k, B[k][j] in lane j + 16 k, D[i][j] in lane j + 16 (i % 4),
// element i / 4); the Cholesky with its retries and the triangular solves run
// on the vector units from LDS.
//
// A's row stride is mp + P for the P lanes per row of the substitutions: the 16
// lanes an LDS access serves per cycle (rows b.. and their P columns) then fall
// in distinct banks.  L keeps stride mp + 1, which the lane-per-row Cholesky
// reads without conflicts.
__host__ __device__ constexpr int gram_lda(int mp) { return mp <= 16 ? mp + 4 : (mp <= 32 ? mp + 2 : mp + 4); }

// Forward then back substitution with the Cholesky factor L (row stride ld)
// for every row b < m of X (row stride ldx), in place: X[b] <- (L L^T)^-1 X[b],
// with inv[i] = 1 / L[i][i].  P lanes share a row: each sums every P-th term of
// a step's dot product, the P partial sums are added across the lanes (an
// aligned lane group of one wave), and the group's first lane stores the step's
// result, which later steps read back from LDS (the LDS operations of a wave
// complete in order).
template <int P>
__device__ void solve_rows(double *X, int ldx, const double *L, int ld, const double *inv, int m, int tid)
{
    static_assert(P >= 1 && P <= 16 && (P & (P - 1)) == 0, "lane group within a DPP row");
    const int b = tid / P, sub = tid % P;
    if (b >= m) return;  // whole lane groups leave together
    double *x = X + (size_t)b * ldx;
    for (int i = 0; i < m; ++i) {
        double part = 0.0;
#pragma unroll 4
        for (int k = sub; k < i; k += P) part = fma(L[i * ld + k], x[k], part);
        const double tot = P > 1 ? group_sum<P>(part) : part;
        if (sub == 0) x[i] = (x[i] - tot) * inv[i];
        __builtin_amdgcn_wave_barrier();
    }
    for (int i = m - 1; i >= 0; --i) {
        double part = 0.0;
#pragma unroll 4
        for (int k = i + 1 + sub; k < m; k += P) part = fma(L[k * ld + i], x[k], part);
        const double tot = P > 1 ? group_sum<P>(part) : part;
        if (sub == 0) x[i] = (x[i] - tot) * inv[i];
        __builtin_amdgcn_wave_barrier();
    }
}

// Eight waves per SIMD (at most 64 registers): with two matrices of LDS per
// head, eight work-groups of the m <= 32 shapes fit on a CU.
__global__ __launch_bounds__(kThreads, 8) void gram_pinv_kernel(DevState s, PrefillIO io, double ridge_rel)
{
    const int H = s.hpk, ci = blockIdx.x / H, h = blockIdx.x - ci * H;
    const size_t gh = (size_t)io.map.state(ci) * H + h;  // state head
    const int m = s.m, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nb = (m + 15) / 16, mp = nb * 16, ld = mp + 1, lda = gram_lda(mp);
    extern __shared__ double lds[];
    double *A = lds;                      // exp-Gram; then row b holds column b of M
    double *L = lds + (size_t)mp * lda;   // G = A^T A + lambda I, factored in place
    __shared__ double mean_diag_s;
    __shared__ int fail_s;
    __shared__ double inv_s[kMaxLandmarks];

    const int li = lane & 15, lk = lane >> 4;
    // the exp-Gram of this head from the landmark kernel, zero-padded to mp x mp
    const double *a64 = io.a64 + ((size_t)ci * H + h) * m * m;
    for (int t = tid; t < mp * mp; t += kThreads) {
        const int i = t / mp, j = t - i * mp;
        A[i * lda + j] = (i < m && j < m) ? a64[i * m + j] : 0.0;
    }
    __syncthreads();
    // G = A^T A into L (padding rows of A are zero).  G is not kept apart from
    // its factor: a retry recomputes it, bit for bit, from A.
    auto gram = [&]() {
        for (int blk = wave; blk < nb * nb; blk += kThreads / 64) {
            const int bi = blk / nb, bj = blk - bi * nb;
            f64x4 acc = {0.0, 0.0, 0.0, 0.0};
            for (int ks = 0; ks < mp / 4; ++ks)
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64(A[(ks * 4 + lk) * lda + bi * 16 + li],
                                                          A[(ks * 4 + lk) * lda + bj * 16 + li], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) L[(bi * 16 + lk + 4 * r) * ld + bj * 16 + li] = acc[r];
        }
    };
    gram();
    __syncthreads();
    if (tid == 0) {
        double md = 0.0;
        for (int i = 0; i < m; ++i) md += L[i * ld + i];
        mean_diag_s = md / (double)m;
    }
    __syncthreads();
    const double floor_diag = mean_diag_s > DBL_MIN ? mean_diag_s : DBL_MIN;
    double lambda = ridge_rel * floor_diag;
    int result = kRidgeTries + 1;

    for (int attempt = 1; attempt <= kRidgeTries; ++attempt) {
        if (attempt > 1) {
            gram();
            __syncthreads();
        }
        for (int i = tid; i < m; i += kThreads) L[i * ld + i] += lambda;  // G + lambda I
        __syncthreads();
        if (wave == 0) {
            // Left-looking Cholesky in one wave, lane i owning row i: for column
            // j every lane i >= j forms s_i = L[i][j] - sum_{k<j} L[i][k] L[j][k];
            // lane j's s is the pivot (a failed pivot is <= 0 or not finite).
            int bad = 0;
            for (int j = 0; j < m; ++j) {
                double sv = 0.0;
                if (lane >= j && lane < m) {
                    double v = L[lane * ld + j];
                    // unrolled so eight steps' LDS reads are in flight; the
                    // subtractions keep their order
#pragma unroll 8
                    for (int k = 0; k < j; ++k) v -= L[lane * ld + k] * L[j * ld + k];
                    sv = v;
                }
                const double p = lane_value(sv, j);
                if (!(p > 0.0) || !isfinite(p)) {
                    bad = 1;
                    break;
                }
                const double dj = sqrt(p);
                if (lane == j) L[j * ld + j] = dj;
                else if (lane > j && lane < m) L[lane * ld + j] = sv / dj;
                __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
            }
            if (lane == 0) fail_s = bad;
        }
        __syncthreads();
        const int failed = fail_s;
        __syncthreads();
        if (!failed) {
            result = attempt;
            break;
        }
        lambda *= 10.0;
    }

    float *mu = s.mu + gh * m * m;
    if (result <= kRidgeTries) {
        for (int i = tid; i < m; i += kThreads) inv_s[i] = 1.0 / L[i * ld + i];
        __syncthreads();
        // Column b of M solves (L L^T) x = (row b of A), in place in row b.
        // one wave (P * mp = 64) while m <= 32, four lanes per row over the
        // whole work-group beyond (measured best of the two at each size)
        if (mp <= 16) solve_rows<4>(A, lda, L, ld, inv_s, m, tid);
        else if (mp <= 32) solve_rows<2>(A, lda, L, ld, inv_s, m, tid);
        else solve_rows<4>(A, lda, L, ld, inv_s, m, tid);
        __syncthreads();
        for (int t = tid; t < m * m; t += kThreads) {
            const int a = t / m, b = t - a * m;
            mu[t] = (float)A[(size_t)b * lda + a];
        }
    } else {
        for (int t = tid; t < m * m; t += kThreads) {
            const int a = t / m, b = t - a * m;
            mu[t] = (a == b) ? (float)(1.0 / floor_diag) : 0.0f;
        }
    }
    if (tid == 0) {
        s.lambda[gh] = lambda;
        s.tries[gh] = result;
    }
}

// ---- far field of the prompt on the matrix cores ---------------------------
//
// One work-group per (group, block of HB heads): the far keys' K and V tiles are
// loaded once and used by every head of the block, and the head blocks of one
// group run on one XCD (work-group b goes to XCD b mod 8), so they share its L2.
// One wave per 16-landmark row block of one head, its Q~ rows held in registers.
// Every product is taken transposed, so that each lane owns one landmark row
// (row li = lane % 16 of the wave's block) throughout:
//   L^T = K_tile Q~_blk^T * scale     keys x rows, D/4 MFMA 16x16x4 f64; lane
//                                     holds keys 4 e + lk (lk = lane / 16) of row li
//   row max: in the lane over its 4 keys, then across lk (lane ^ 16, ^ 32)
//   P   = e^{L - max} in f32 (the gap is formed in f64; at most 1 in value, so
//         its absolute error is that of an f32 rounding), Z^ += row sums (f64)
//   T^T <- T^T * e^{max_old - max_new} + V_tile^T P^T    dv x rows, 4 * dv/16
//         MFMA 16x16x4 f32; P's operand for k-step kk is this lane's own weight
//         e = kk (key 4 kk + lk), so P never leaves the registers
// The logit product runs over a permuted component order: at step ks, lane
// (i, k) holds K[i][k * D/4 + ks] and Q~[i][k * D/4 + ks], so each lane's Q~
// operands are one contiguous run of D/4 components and the sum over k and ks
// still covers every component once.
// Operand layout of both MFMAs (wave64): A[i][k] in lane i + 16 k, B[k][j] in
// lane j + 16 k; results: f64 D[i][j] in lane j + 16 (i % 4), element i / 4; f32
// D[i][j] in lane j + 16 (i / 4), element i % 4.

typedef float f32x4 __attribute__((ext_vector_type(4)));

// x + x(lane ^ 16) + x(lane ^ 32) + x(lane ^ 48): the four lanes of one row
// index li (f32, exact exchanges as in sum_high_lanes)
__device__ __forceinline__ float sum_over_lk(float x)
{
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// (At least two waves per SIMD: otherwise a 4-wave work-group may take the
// whole register file, and one work-group per CU leaves the MFMAs idle on loads.)
template <int D, int DV, int MM, int HB>
__global__ __launch_bounds__(64 * HB * (MM / 16), 2) void far_mfma_kernel(DevState s, PrefillIO io)
{
    constexpr int NRB = MM / 16, NW = HB * NRB, NT = 64 * NW;
    constexpr int KS = D / 4;    // k-steps of the logit product = components per lane
    constexpr int CB = DV / 16;  // 16-wide column blocks of T^
    constexpr int TK = 16;       // keys per tile
    constexpr int K4 = TK * (D / 4), KV4 = K4 + TK * (DV / 4);  // float4 of a K tile, of K and V
    constexpr int PT = (KV4 + NT - 1) / NT;                     // float4 per thread per tile
    constexpr int VLD = DV + 16;  // V tile row stride (floats): the 4 rows an operand read touches start 16 banks apart
    constexpr double LOG2E = 1.4426950408889634;
    const int H = s.hpk, nhb = (H + HB - 1) / HB;
    const int jb = blockIdx.x >> 3;
    const int ci = (jb / nhb) * 8 + (blockIdx.x & 7), hb = jb - (jb / nhb) * nhb;
    if (ci >= io.map.count) return;
    const int g = io.map.state(ci);
    const int m = s.m, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = hb * HB + wave / NRB, rb = wave % NRB;
    const bool live = h < H && rb * 16 < m;  // waves past hpk or m hold no rows
    const size_t gh = (size_t)g * H + min(h, H - 1);
    const int S = s.sink, nf = io.T - S - s.w;
    const double sc = (double)s.scale;
    const double NEG_INF = -__builtin_inf();
    const int li = lane & 15, lk = lane >> 4;

    // K tiles widened to f64 once, as they are staged: the MFMA operand reads
    // need no conversion.  K is [k quarter][key][component] with an odd row
    // length, so the 16 keys of an operand read fall in distinct bank pairs.
    // V stays f32 (the weights' product runs on f32 MFMA).
    __shared__ double k_lds[4][TK][KS + 1];
    __shared__ float v_lds[TK][VLD];

    // Q~ fragment of this wave: row rb * 16 + li, components lk * KS .. lk * KS + KS - 1
    float qa[KS];
    {
        const int row = rb * 16 + li;
        const float4 *src =
            reinterpret_cast<const float4 *>(s.q_tilde + (gh * m + min(row, m - 1)) * D + lk * KS);
        const bool use = live && row < m;
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            const float4 x = src[c];
            qa[4 * c + 0] = use ? x.x : 0.0f;
            qa[4 * c + 1] = use ? x.y : 0.0f;
            qa[4 * c + 2] = use ? x.z : 0.0f;
            qa[4 * c + 3] = use ? x.w : 0.0f;
        }
    }

    // K and V tiles: thread slot p covers float4 tid + p * NT of [K tile | V tile];
    // key indices are clamped (dead keys get zero weights below)
    const float *K = io.p.k_row(io.map, ci, S);
    const float *V = io.p.v_row(io.map, ci, S);
    const int64_t kpos = io.p.k_pos, vpos = io.p.v_pos;
    float4 pre[PT];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int idx = min(tid + p * NT, KV4 - 1);
            const bool isk = idx < K4;
            const int e = isk ? idx : idx - K4, per = isk ? D / 4 : DV / 4;
            const int key = min(j0 + e / per, nf - 1), c4 = e % per;
            const float *row = isk ? K + (int64_t)key * kpos : V + (int64_t)key * vpos;
            pre[p] = reinterpret_cast<const float4 *>(row)[c4];
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int idx = tid + p * NT;
            if (idx < K4) {
                const int key = idx / (D / 4), c = (idx % (D / 4)) * 4;  // component of .x
                double *dst = &k_lds[c / KS][key][c % KS];
                dst[0] = pre[p].x;
                dst[1] = pre[p].y;
                dst[2] = pre[p].z;
                dst[3] = pre[p].w;
            } else if (idx < KV4) {
                const int e = idx - K4, key = e / (DV / 4), c4 = e % (DV / 4);
                *reinterpret_cast<float4 *>(&v_lds[key][c4 * 4]) = pre[p];
            }
        }
    };

    f32x4 tacc[CB];  // T^ transposed: element e of lane (li, lk) is column 4 lk + e of row li
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) tacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    double mx = NEG_INF, zs = 0.0;  // row li: running max, Z^

    fetch(0);
    for (int j0 = 0; j0 < nf; j0 += TK) {
        const int nt = min(TK, nf - j0);
        stage();
        __syncthreads();
        if (j0 + TK < nf) fetch(j0 + TK);  // the next tile is in flight during the MFMAs

        // logits of the tile against this landmark block, transposed
        f64x4 L = {0.0, 0.0, 0.0, 0.0}, L2 = {0.0, 0.0, 0.0, 0.0}, L3 = L, L4 = L;
#pragma unroll
        for (int ks = 0; ks < KS; ks += 4) {
            // opaque copies: widen Q~ at its use instead of keeping KS doubles live
            float q0 = qa[ks], q1 = qa[ks + 1], q2 = qa[ks + 2], q3 = qa[ks + 3];
            asm volatile("" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3));
            L = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks], (double)q0, L, 0, 0, 0);
            L2 = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks + 1], (double)q1, L2, 0, 0, 0);
            L3 = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks + 2], (double)q2, L3, 0, 0, 0);
            L4 = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks + 3], (double)q3, L4, 0, 0, 0);
        }
        L = (L + L2) + (L3 + L4);
        // lane holds L[key 4 e + lk][row li], e = 0..3
        double l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) l[e] = 4 * e + lk < nt ? L[e] * sc : NEG_INF;
        double rmax = fmax(fmax(l[0], l[1]), fmax(l[2], l[3]));
        rmax = swap_max<32>(swap_max<16>(rmax));  // row li over the whole tile
        const double nw = fmax(mx, rmax);
        if (__any(nw != mx)) {  // rescale only when some running max of the wave moved
            const double f = exp(mx - nw);  // 0 on the first tile, 1 where the max held
            zs *= f;
            const float ff = (float)f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) tacc[cb] *= ff;
        }
        mx = nw;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            p[e] = 4 * e + lk < nt ? __builtin_amdgcn_exp2f((float)((l[e] - nw) * LOG2E)) : 0.0f;
        zs += (double)sum_over_lk((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // consecutive MFMAs go to different accumulators
            float va[CB];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) va[cb] = v_lds[kk * 4 + lk][cb * 16 + li];
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                tacc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(va[cb], p[kk], tacc[cb], 0, 0, 0);
        }
        __syncthreads();  // every wave is done with the tile before the next is staged
    }

    if (!live) return;
    // store at the scale of the f32 running max kept in the state
    const int i = rb * 16 + li;
    if (i >= m) return;
    const float mf = (float)mx;
    const double corr = exp(mx - (double)mf);
    if (lk == 0) {
        s.m_max[gh * m + i] = mf;
        s.m_ref[gh * m + i] = mf;
        s.z_hat[gh * m + i] = zs * corr;
    }
    float4 *th = reinterpret_cast<float4 *>(s.t_hat + (gh * m + i) * DV);
    const float cf = (float)corr;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
        th[cb * 4 + lk] = make_float4(tacc[cb][0] * cf, tacc[cb][1] * cf, tacc[cb][2] * cf, tacc[cb][3] * cf);
}

template <int D, int DV, int MM>
hipError_t launch_far(const DevState &s, const PrefillIO &io, hipStream_t stream)
{
    // heads per work-group: as many as keep it at 512 threads or fewer
    constexpr int HB_MAX = 8 / (MM / 16);
    int hb = HB_MAX;  // a power of two; the last block of a group may hold fewer heads
    while (hb > s.hpk) hb /= 2;
    const long long nhb = (s.hpk + hb - 1) / hb;
    const long long grid = 8LL * nhb * ((io.map.count + 7) / 8);
    switch (hb) {
    case 1: hipLaunchKernelGGL((far_mfma_kernel<D, DV, MM, 1>), dim3((unsigned)grid), dim3(64 * MM / 16), 0, stream, s, io); break;
    case 2: hipLaunchKernelGGL((far_mfma_kernel<D, DV, MM, 2>), dim3((unsigned)grid), dim3(128 * MM / 16), 0, stream, s, io); break;
    case 4:
        if constexpr (HB_MAX >= 4) {
            hipLaunchKernelGGL((far_mfma_kernel<D, DV, MM, 4>), dim3((unsigned)grid), dim3(256 * MM / 16), 0, stream, s, io);
            break;
        }
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_far_m(const DevState &s, const PrefillIO &io, hipStream_t stream)
{
    if (s.m <= 32) return launch_far<D, DV, 32>(s, io, stream);
    return launch_far<D, DV, 64>(s, io, stream);
}

// Frozen M, [count][hpk][m][m] in call order, into the mapped groups' state.
__global__ void copy_mu_kernel(DevState s, GroupMap map, const float *src)
{
    const size_t per_g = (size_t)s.hpk * s.m * s.m;
    const size_t n = (size_t)map.count * per_g;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (size_t)gridDim.x * blockDim.x) {
        const size_t ci = t / per_g;
        s.mu[(size_t)map.state((int)ci) * per_g + (t - ci * per_g)] = src[t];
    }
    const size_t nh = (size_t)map.count * s.hpk;
    for (size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x; t < nh; t += (size_t)gridDim.x * blockDim.x) {
        const size_t ci = t / s.hpk;
        const size_t gh = (size_t)map.state((int)ci) * s.hpk + (t - ci * s.hpk);
        s.lambda[gh] = 0.0;
        s.tries[gh] = 0;
    }
}

}  // namespace

hipError_t launch_prefill(const DevState &s, const PrefillIO &io, hipStream_t stream)
{
    if (s.d > 128 || s.dv > 128 || s.m > kMaxLandmarks) return hipErrorInvalidValue;
    const int n = io.map.count;
    const int mp = (s.m + 15) / 16 * 16;
    const size_t lm_lds = sizeof(double) * 2 * mp * (s.d + 1);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&landmarks_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lm_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(landmarks_kernel, dim3(n), dim3(kLmThreads), lm_lds, stream, s, io, io.fz_mu ? 0 : 1);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(n), dim3(kThreads), 0, stream, s, io);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (io.fz_mu) {
        hipLaunchKernelGGL(copy_mu_kernel, dim3(1024), dim3(kThreads), 0, stream, s, io.map, io.fz_mu);
    } else {
        const size_t lds = sizeof(double) * mp * (gram_lda(mp) + mp + 1);
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&gram_pinv_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(gram_pinv_kernel, dim3(n * s.hpk), dim3(kThreads), lds, stream, s, io, io.ridge_rel);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // far-insert logits of the ring's keys (the landmarks and ring are in place)
    if ((err = launch_ring_logits(s, io.map, stream)) != hipSuccess) return err;
    if (s.d == 128 && s.dv == 128) return launch_far_m<128, 128>(s, io, stream);
    if (s.d == 64 && s.dv == 64) return launch_far_m<64, 64>(s, io, stream);
    return hipErrorInvalidValue;
}

}  // namespace o1
