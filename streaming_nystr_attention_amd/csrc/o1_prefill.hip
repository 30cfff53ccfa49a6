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
//   gram_pinv_kernel   one wave per 64 / mp heads (mp = m rounded up to 16),
//                      a lane per matrix row: G = A^T A on f64 MFMA from the
//                      exp-Gram, lambda = ridge_rel * max(mean diag G, DBL_MIN),
//                      Cholesky of G + lambda I with the rows in registers
//                      (lambda x10 on a failed pivot, up to 12 attempts, then
//                      diag(1/mean diag)), M = (G + lambda I)^-1 A^T by forward
//                      and back substitution, a right-hand side per lane.  One
//                      mp x (mp + 1) f64 matrix of LDS per head.
//   ring_logits_kernel grid G * hpk / hb: the far-insert logits of every ring
//                      slot's key against each head's query landmarks (kept per
//                      slot for the decode's evictions), f64 MFMA with the
//                      landmark queries staged in LDS; also run after state writes.
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
constexpr size_t kLmLdsMax = 132 * 1024;  // dynamic LDS of the landmark pass

// Near-state row of prompt key j, or -1: sinks j < sink keep row j, the last w
// keys go to ring slot (j - sink) mod w (row sink + slot).
__device__ __forceinline__ int near_row(int j, int S, int w, int T)
{
    if (j < S) return j;
    if (j >= T - w) return S + (j - S) % w;
    return -1;
}

// Segment means of columns c0 .. c0 + dc - 1 of the rows of x (row stride pos
// floats) into dst32 (state, f32, row length d) and l64 (LDS, f64, row stride
// ld, column c0 at 0): one thread per (segment, 4 components), the segment's
// rows summed in row order, eight rows' loads in flight at a time.  With
// `near`, the chunk's columns of rows that are sinks or ring keys are also
// copied there.
__device__ __forceinline__ void seg_means_pass(const float *x, int64_t pos, int T, int m, int d, int c0,
                                               int dc, float *dst32, double *l64, int ld, float4 *near,
                                               int S, int w)
{
    const int d4 = d / 4, dc4 = dc / 4;
    for (int t = threadIdx.x; t < m * dc4; t += kLmThreads) {
        const int a = t / dc4, cl = (t - a * dc4) * 4, c = c0 + cl, c4 = c / 4;
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
            l64[a * ld + cl + e] = mean[e];
            dst32[a * d + c + e] = (float)mean[e];
        }
    }
}

// Frozen landmarks given by the caller, columns c0 .. c0 + dc - 1: the state
// takes them, LDS their f64 values.
__device__ __forceinline__ void frozen_pass(const float *fz, int m, int d, int c0, int dc, float *dst32,
                                            double *l64, int ld)
{
    for (int t = threadIdx.x; t < m * dc; t += kLmThreads) {
        const int a = t / dc, cl = t - a * dc;
        const float v = fz[a * d + c0 + cl];
        dst32[a * d + c0 + cl] = v;
        l64[a * ld + cl] = (double)v;
    }
}

// One work-group per group, 512 threads (two per CU, as LDS allows at m <= 32,
// d = 128: four waves per SIMD); dynamic LDS: K~ and one head's Q~ in f64,
// [mp][dc + 1] each (mp = m rounded up to 16, rows past m zero) for a chunk of
// dc of the d components.  The exp-Gram of head h, A[i][j] = exp(q~_i . k~_j
// * scale), runs on v_mfma_f64_16x16x4f64 from LDS, one 16 x 16 block per wave,
// and goes to io.a64[call][h][mp][mp], zero past m, for gram_pinv_kernel
// (`gram` = 0: M is given frozen and no A is needed).  When both [mp][d + 1]
// arrays do not fit (d = 256, m > 32) the components come in chunks (dc = d /
// 2): each chunk's key pass, then each head's query pass and the dots over
// the chunk, the partial dots kept in io.a64 until the last chunk takes the
// exp.  Every prompt row is still read once.
__global__ __launch_bounds__(kLmThreads, 4) void landmarks_kernel(DevState s, PrefillIO io, int gram, int dc)
{
    const int ci = blockIdx.x, g = io.map.state(ci);
    const int d = s.d, m = s.m, T = io.T, H = s.hpk, tid = threadIdx.x;
    const int nb = (m + 15) / 16, mp = nb * 16, ld = dc + 1, nch = d / dc;
    extern __shared__ double lm_lds[];
    double *kt64 = lm_lds, *qt64 = lm_lds + (size_t)mp * ld;
    // rows past m stay zero for every head and chunk
    for (int t = tid; t < (mp - m) * ld; t += kLmThreads) {
        kt64[m * ld + t] = 0.0;
        qt64[m * ld + t] = 0.0;
    }

    float *kt32 = s.k_tilde + (size_t)g * m * d;
    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    const double sc = (double)s.scale;
    for (int ch = 0; ch < nch; ++ch) {
        const int c0 = ch * dc;
        const bool first = ch == 0, last = ch == nch - 1;
        __syncthreads();  // the previous chunk's dots are done with kt64
        if (io.fz_kt) {
            frozen_pass(io.fz_kt + (size_t)ci * m * d, m, d, c0, dc, kt32, kt64, ld);
        } else {
            float4 *near = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * s.R * (d / 4);
            seg_means_pass(io.p.k_row(io.map, ci, 0), io.p.k_pos, T, m, d, c0, dc, kt32, kt64, ld, near,
                           s.sink, s.w);
        }
        for (int h = 0; h < H; ++h) {
            float *qt32 = s.q_tilde + ((size_t)g * H + h) * m * d;
            __syncthreads();  // the previous head's exp-Gram is done with qt64
            if (io.fz_qt)
                frozen_pass(io.fz_qt + ((size_t)ci * H + h) * m * d, m, d, c0, dc, qt32, qt64, ld);
            else
                seg_means_pass(io.p.q_row(io.map, H, ci, h, 0), io.p.q_pos, T, m, d, c0, dc, qt32, qt64, ld,
                               nullptr, 0, 0);
            if (!gram) continue;
            __syncthreads();
            double *a = io.a64 + ((size_t)ci * H + h) * mp * mp;
            for (int blk = wave; blk < nb * nb; blk += kLmThreads / 64) {
                const int bi = blk / nb, bj = blk - bi * nb;
                const double *qrow = qt64 + (bi * 16 + li) * ld + lk;
                const double *krow = kt64 + (bj * 16 + li) * ld + lk;
                f64x4 acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
                // k-step ks covers components 4 ks .. 4 ks + 3 (k-lane lk: 4 ks + lk)
                for (int ks = 0; ks < dc / 4; ks += 2) {
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qrow[4 * ks], krow[4 * ks], acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(qrow[4 * ks + 4], krow[4 * ks + 4], acc2, 0, 0, 0);
                }
                acc += acc2;
                // lane holds A[bi*16 + lk + 4 r][bj*16 + li]; this thread wrote
                // the same entries for the earlier chunks
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = bi * 16 + lk + 4 * r, j = bj * 16 + li;
                    const double dot = first ? acc[r] : acc[r] + a[i * mp + j];
                    a[i * mp + j] = (i < m && j < m) ? (last ? exp(dot * sc) : dot) : 0.0;
                }
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

// Value of lane u * MP + j (head u's lane j) in every lane of head u = sub.
template <int MP, int HPW>
__device__ __forceinline__ double head_lane_value(double v, int j, int sub)
{
    double r = lane_value(v, j);
#pragma unroll
    for (int u = 1; u < HPW; ++u) r = sub == u ? lane_value(v, u * MP + j) : r;
    return r;
}

// HPW = 64 / MP heads per wave, one lane per matrix row: a head's ridge
// pseudo-inverse needs no more than MP lanes (m <= 64), so the heads run
// without work-group barriers and interleave on the SIMDs.  MP = m rounded up
// to 16; each matrix is padded to MP x MP as [G 0; 0 I], whose factor is
// [L 0; 0 I] and whose padding adds nothing to the solves.  One MP x (MP + 1)
// f64 matrix of LDS per head holds G, then L^T.
//
//   G = A^T A         per head, all lanes: v_mfma_f64_16x16x4f64 straight from
//                     the exp-Gram in global memory, stored MP x MP with zeros
//                     past m, so every load is unconditional (operand layout:
//                     A[i][k] in lane i + 16 k, B[k][j] in lane j + 16 k,
//                     D[i][j] in lane j + 16 (i % 4), element i / 4); blocks on
//                     and above the diagonal, each stored with its mirror.  Lane
//                     i of the head reads row i into registers.
//   Cholesky          right-looking, as the page's cholesky: the pivot of
//                     column j is the head's lane j's entry j after the updates
//                     of columns 0..j-1 (a pivot not > 0 or not finite fails the
//                     attempt: lambda x10, G recomputed bit for bit from A, up to
//                     12 attempts); lane i divides its entry j by the pivot's
//                     root and stores it as L^T[j][i], then subtracts
//                     L[i][j] L[k][j] (read back from LDS) from its entry k for
//                     k > j.  Heads of a wave retry independently: the lanes of a
//                     head that is done run the later attempts too, but store
//                     into a spare row, so its factor stays.
//   M = (G + lambda I)^-1 A^T
//                     lane b solves (L L^T) x = (row b of A) by forward and back
//                     substitution, x in registers, L from LDS (the same address
//                     in every lane of a head); x is column b of M.
// Loops run over the compile-time MP, fully unrolled, so rows stay in registers;
// after each solve row an empty asm statement that takes the row's result and
// clobbers memory keeps the next row's LDS reads behind it (else every read of
// the solve is hoisted to its start and the registers spill).
template <int MP>
__global__ __launch_bounds__(64) void gram_pinv_kernel(DevState s, PrefillIO io, double ridge_rel)
{
    static_assert(MP % 16 == 0 && MP <= 64, "one lane per row");
    constexpr int HPW = 64 / MP, NB = MP / 16, KS = MP / 4, LD = MP + 1;
    __shared__ double Ws[HPW][(MP + 1) * LD];  // G, then L^T (row j: column j of L); row MP spare
    __shared__ double inv_s[HPW][MP + 1];      // 1 / L[j][j]; entry MP spare
    const int H = s.hpk, nh = io.map.count * H, m = s.m;
    const int lane = threadIdx.x, li = lane & 15, lk = lane >> 4;
    const int sub = min(lane / MP, HPW - 1), row = lane % MP;  // head in the wave, matrix row
    // lanes past HPW * MP (MP = 48) shadow a row of head 0 and store nothing
    const int hidx = blockIdx.x * HPW + sub;  // call-major head index
    const bool owner = lane < HPW * MP && hidx < nh;
    const double *a_of = io.a64 + (size_t)blockIdx.x * HPW * MP * MP;  // zero past m
    const double *a64 = a_of + (size_t)min(sub, nh - 1 - (int)blockIdx.x * HPW) * MP * MP;
    double *W = Ws[sub];

    // G of head u of this wave (heads past the last one recompute the last)
    auto gram = [&](int u) {
        const double *au = a_of + (size_t)min(u, nh - 1 - (int)blockIdx.x * HPW) * MP * MP;
        double av[NB][KS];  // A[4 ks + lk][16 b + li]
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) av[bi][ks] = au[(4 * ks + lk) * MP + 16 * bi + li];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int bj = bi; bj < NB; ++bj) {
                f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[bi][ks], av[bj][ks], acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * bi + lk + 4 * r, j = 16 * bj + li;
                    Ws[u][i * LD + j] = acc[r];
                    Ws[u][j * LD + i] = acc[r];
                }
            }
        asm volatile("" ::: "memory");  // the next head's operands load after these
    };
#pragma unroll
    for (int u = 0; u < HPW; ++u) gram(u);
    __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
    constexpr int GS = HPW * MP == 64 ? MP : 64;  // lanes summed per head
    const double mean_diag =
        group_sum<GS>(lane < HPW * MP && row < m ? W[row * LD + row] : 0.0) / (double)m;
    const double floor_diag = mean_diag > DBL_MIN ? mean_diag : DBL_MIN;
    double lambda = ridge_rel * floor_diag;
    int result = kRidgeTries + 1;
    bool done = false;

#pragma unroll 1
    for (int attempt = 1; attempt <= kRidgeTries; ++attempt) {
        if (attempt > 1) {
#pragma unroll
            for (int u = 0; u < HPW; ++u)
                if (!__builtin_amdgcn_readlane((int)done, u * MP)) gram(u);  // heads still failing
            __builtin_amdgcn_wave_barrier();
        }
        // G + lambda I on the m x m block, 1 on the padding diagonal
        double Lr[MP];
#pragma unroll
        for (int k = 0; k < MP; ++k) {
            const double gk = W[row * LD + k];
            Lr[k] = k != row ? gk : (row < m ? gk + lambda : 1.0);
        }
        __builtin_amdgcn_wave_barrier();  // G read before L^T overwrites it
        // a failed pivot clears `ok` and the factorization runs on with a
        // unit pivot (no branch inside the unrolled steps; the result is
        // discarded); a head already done stores into the spare row
        bool ok = true;
#pragma unroll
        for (int j = 0; j < MP; ++j) {
            const double p = head_lane_value<MP, HPW>(Lr[j], j, sub);
            ok = ok && p > 0.0 && isfinite(p);
            const double dj = sqrt(ok ? p : 1.0);
            const double c = row == j ? dj : Lr[j] / dj;  // L[row][j]
            const int jr = done ? MP : j;
            W[jr * LD + row] = c;
            inv_s[sub][jr] = 1.0 / dj;
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = j + 1; k < MP; ++k) {
                Lr[k] = fma(-c, W[j * LD + k], Lr[k]);
                asm volatile("" : "+v"(Lr[k]));  // updated within step j
            }
            asm volatile("" ::: "memory");
        }
        if (!done && ok) result = attempt;
        done = done || ok;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        if (!done) lambda *= 10.0;
        __builtin_amdgcn_wave_barrier();
    }

    float *mu = s.mu + ((size_t)io.map.state(min(hidx, nh - 1) / H) * H + min(hidx, nh - 1) % H) * m * m;
    const bool fallback = result > kRidgeTries;
    double x[MP];  // row `row` of A: the right-hand side of column `row` of M
#pragma unroll
    for (int k = 0; k < MP; ++k) x[k] = a64[row * MP + k];
#pragma unroll
    for (int i = 0; i < MP; ++i) {
        double tot = 0.0;
#pragma unroll
        for (int k = 0; k < i; ++k) {
            tot = fma(W[k * LD + i], x[k], tot);  // L[i][k]
            if (k % 16 == 15) asm volatile("" : "+v"(tot)::"memory");  // 16 reads in flight
        }
        x[i] = (x[i] - tot) * inv_s[sub][i];
        asm volatile("" : "+v"(x[i])::"memory");
    }
#pragma unroll
    for (int i = MP - 1; i >= 0; --i) {
        double tot = 0.0;
#pragma unroll
        for (int k = i + 1; k < MP; ++k) {
            tot = fma(W[i * LD + k], x[k], tot);  // L[k][i]
            if ((k - i) % 16 == 0) asm volatile("" : "+v"(tot)::"memory");  // 16 reads in flight
        }
        x[i] = (x[i] - tot) * inv_s[sub][i];
        asm volatile("" : "+v"(x[i])::"memory");
    }
    // column `row` of M; a head whose attempts all failed takes diag(1 / mean diag)
    if (owner && row < m) {
        const float fb = (float)(1.0 / floor_diag);
#pragma unroll
        for (int a = 0; a < MP; ++a)
            if (a < m) mu[a * m + row] = fallback ? (a == row ? fb : 0.0f) : (float)x[a];
        if (row == 0) {
            const size_t gh = (size_t)io.map.state(hidx / H) * H + hidx % H;
            s.lambda[gh] = lambda;
            s.tries[gh] = result;
        }
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

// Occupancy: the MFMAs of one wave's tile are a dependent chain, so they stay
// busy only with other waves to switch to.  Work-groups of four waves run at
// three waves per SIMD (three work-groups per CU), those of eight at four (two
// per CU; a few address registers spill), with the logits summed in two
// accumulator chains to fit; two-wave work-groups (one head of m <= 32) and
// rows of 256 floats, whose tiles need more registers, at two per SIMD.
template <int D, int DV, int MM, int HB>
__global__ __launch_bounds__(64 * HB * (MM / 16), (D > 128 || HB * (MM / 16) == 2 ? 2 : (HB * (MM / 16) == 4 ? 3 : 4))) void far_mfma_kernel(DevState s, PrefillIO io)
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
        f64x4 L = {0.0, 0.0, 0.0, 0.0}, L2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int ks = 0; ks < KS; ks += 2) {
            // opaque copies: widen Q~ at its use instead of keeping KS doubles live
            float q0 = qa[ks], q1 = qa[ks + 1];
            asm volatile("" : "+v"(q0), "+v"(q1));
            L = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks], (double)q0, L, 0, 0, 0);
            L2 = __builtin_amdgcn_mfma_f64_16x16x4f64(k_lds[lk][li][ks + 1], (double)q1, L2, 0, 0, 0);
        }
        L = L + L2;
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

// One work-group (4 waves) per (call index, block of hb heads): the far-insert
// logits of every ring slot's key, ring_l[g][s][h][i] = q~_{h,i} . k_{sink+s} * scale,
// a dense [w x d] x [d x m] product per head on f64 MFMA (v_mfma_f64_16x16x4f64:
// f32 inputs widened to f64, so every product is exact and the sums are f64).
// The block's landmark queries (hb * m rows) are staged in LDS once; each wave
// holds one 16-slot tile of ring keys (A) in registers, loaded straight from
// global memory, and walks the landmark tiles of its heads (B) from LDS.  The
// reduction index is permuted so that the four k-lanes of a row read 64
// contiguous bytes: in MFMA step (j, c), k-lane kk stands for column
// 16 j + 4 kk + c, for A and B alike.  Rows past w or m are clamped to the last
// row; their products reach only outputs that are not stored.
// Operand layout: A[i][k] in lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in
// lane j + 16 (i mod 4), element i / 4.
template <int D>
__global__ __launch_bounds__(256) void ring_logits_kernel(DevState s, GroupMap map, int hb)
{
    constexpr int NJ = D / 16, D4 = D / 4, LDQ = D4 + 1;  // LDS row stride (float4): rows start 4 banks apart
    extern __shared__ float4 qt_s[];                      // [hb * m][LDQ]
    const int g = map.state(blockIdx.x), h0 = blockIdx.y * hb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    const int m = s.m, w = s.w, H = s.hpk;
    const int st = (w + 15) / 16, mt = (m + 15) / 16, nb = hb * mt;  // slot tiles; (head, landmark tile) pairs
    const float4 *ring = reinterpret_cast<const float4 *>(s.near_k) + ((size_t)g * s.R + s.sink) * D4 + lk;
    const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + ((size_t)g * H + h0) * m * D4;
    const double scale = (double)s.scale;
    using d4v = __attribute__((ext_vector_type(4))) double;

    for (int t = tid; t < hb * m * D4; t += 256) {
        const int r = t / D4, c = t - r * D4;
        qt_s[r * LDQ + c] = qt[t];
    }
    __syncthreads();

    for (int a = wave; a < st; a += 4) {
        float4 x[NJ];
        const float4 *kr = ring + (size_t)min(16 * a + li, w - 1) * D4;
#pragma unroll
        for (int j = 0; j < NJ; ++j) x[j] = kr[4 * j];
        for (int t = 0; t < nb; ++t) {  // head h0 + t / mt, landmark tile t % mt
            const int hh = t / mt, i = 16 * (t - hh * mt) + li;
            const float4 *qr = qt_s + (hh * m + min(i, m - 1)) * LDQ + lk;
            d4v acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float4 y = qr[4 * j];
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[j].x, (double)y.x, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[j].y, (double)y.y, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[j].z, (double)y.z, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[j].w, (double)y.w, acc, 0, 0, 0);
            }
            if (i >= m) continue;
            double *dst = s.ring_l + ((size_t)g * w * H + h0 + hh) * m + i;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = 16 * a + 4 * e + lk;
                if (slot < w) dst[(size_t)slot * H * m] = acc[e] * scale;
            }
        }
    }
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
    if (s.d > 256 || s.dv > 256 || s.m > kMaxLandmarks) return hipErrorInvalidValue;
    const int n = io.map.count;
    const int mp = (s.m + 15) / 16 * 16;
    // K~ and Q~ of the landmark pass as f64 [mp][dc + 1], dc = d unless that
    // passes 132 KB of LDS (d = 256, m > 32), then half the components at a time
    const int dc = sizeof(double) * 2 * mp * (s.d + 1) <= kLmLdsMax ? s.d : s.d / 2;
    const size_t lm_lds = sizeof(double) * 2 * mp * (dc + 1);
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(&landmarks_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lm_lds);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(landmarks_kernel, dim3(n), dim3(kLmThreads), lm_lds, stream, s, io, io.fz_mu ? 0 : 1, dc);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(scatter_kernel, dim3(n), dim3(kThreads), 0, stream, s, io);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (io.fz_mu) {
        hipLaunchKernelGGL(copy_mu_kernel, dim3(1024), dim3(kThreads), 0, stream, s, io.map, io.fz_mu);
    } else {
        // 64 / mp heads per one-wave work-group
        const auto grid = [&](int hpw) { return dim3((unsigned)((n * s.hpk + hpw - 1) / hpw)); };
        switch (mp) {
        case 16: hipLaunchKernelGGL(gram_pinv_kernel<16>, grid(4), dim3(64), 0, stream, s, io, io.ridge_rel); break;
        case 32: hipLaunchKernelGGL(gram_pinv_kernel<32>, grid(2), dim3(64), 0, stream, s, io, io.ridge_rel); break;
        case 48: hipLaunchKernelGGL(gram_pinv_kernel<48>, grid(1), dim3(64), 0, stream, s, io, io.ridge_rel); break;
        default: hipLaunchKernelGGL(gram_pinv_kernel<64>, grid(1), dim3(64), 0, stream, s, io, io.ridge_rel); break;
        }
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // far-insert logits of the ring's keys (the landmarks and ring are in place)
    if ((err = launch_ring_logits(s, io.map, stream)) != hipSuccess) return err;
    if (s.d == 128 && s.dv == 128) return launch_far_m<128, 128>(s, io, stream);
    if (s.d == 96 && s.dv == 96) return launch_far_m<96, 96>(s, io, stream);
    if (s.d == 256 && s.dv == 256) return launch_far_m<256, 256>(s, io, stream);
    if (s.d == 64 && s.dv == 64) return launch_far_m<64, 64>(s, io, stream);
    if (s.d == 192 && s.dv == 128) return launch_far_m<192, 128>(s, io, stream);
    if (s.d == 80 && s.dv == 80) return launch_far_m<80, 80>(s, io, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_ring_logits(const DevState &s, const GroupMap &map, hipStream_t stream)
{
    if (!s.ring_l) return hipSuccess;
    if (s.m < 1 || s.m > kMaxLandmarks || s.w < 1 || s.hpk < 1) return hipErrorInvalidValue;
    // heads per work-group: all of a group's heads (its ring rows loaded once)
    // unless that leaves fewer than 2048 work-groups or stages more than 64
    // landmark rows in LDS
    int hb = s.hpk;
    const int max_rows = s.d > 128 ? 32 : 64;  // landmark rows staged per work-group (33.8 KB)
    while (hb > 1 && ((long)map.count * (s.hpk / hb) < 2048 || hb * s.m > max_rows)) hb /= 2;
    if (s.hpk % hb) hb = 1;
    const dim3 grid(map.count, s.hpk / hb);
    const size_t lds = sizeof(float4) * (size_t)hb * s.m * (s.d / 4 + 1);
    if (lds > 64 * 1024) {  // 64 landmark rows of 256 floats: above the default dynamic limit
        hipError_t err = hipSuccess;
        if (s.d == 256)
            err = hipFuncSetAttribute(reinterpret_cast<const void *>(&ring_logits_kernel<256>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    if (s.d == 64)
        hipLaunchKernelGGL(ring_logits_kernel<64>, grid, dim3(256), lds, stream, s, map, hb);
    else if (s.d == 80)
        hipLaunchKernelGGL(ring_logits_kernel<80>, grid, dim3(256), lds, stream, s, map, hb);
    else if (s.d == 96)
        hipLaunchKernelGGL(ring_logits_kernel<96>, grid, dim3(256), lds, stream, s, map, hb);
    else if (s.d == 128)
        hipLaunchKernelGGL(ring_logits_kernel<128>, grid, dim3(256), lds, stream, s, map, hb);
    else if (s.d == 192)
        hipLaunchKernelGGL(ring_logits_kernel<192>, grid, dim3(256), lds, stream, s, map, hb);
    else if (s.d == 256)
        hipLaunchKernelGGL(ring_logits_kernel<256>, grid, dim3(256), lds, stream, s, map, hb);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace o1
