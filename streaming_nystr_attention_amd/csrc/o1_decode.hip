// One decode step of streaming Nystrom attention for every group: the
// NystromState::step_group of the nystrom.rs source page (advance, then
// NystromHead::step per query head), batched as one work-group per group.
//
// The step reads each group's whole state once, so it is bound by HBM, and a
// work-group's time is mostly memory latency.  The kernel is organised to keep
// few dependent round trips per group and many bytes in flight:
//
//   0. prologue, small loads staged into LDS: the ring head e = win_head, the
//      queries, the new k/v, the evicted ring row (row sink+e), each head's
//      running max and Z^, and (small shapes) each head's mixing matrix M.
//      (Each staging loop waits for its own loads; issuing them all first
//      measured slower on large launches, whose work-groups overlap anyway.)
//      Then row sink+e is overwritten by the new k/v (advance); nothing reads
//      that row from global memory afterwards.
//   1. row-dot pass, f64 accumulation, each row split over LPR lanes and UNR
//      rows per lane in flight:
//        near logits  lg[h][r] = q_h . k_r * scale       (sink + w rows, all heads)
//        landmark     s[h][a]  = q_h . k~_a * scale      (m rows, all heads)
//        far insert   l[h][i]  = q~_{h,i} . k_e * scale  (hpk * m rows)
//      The hpk partial dots of a row are reduced over the row's lanes by
//      halving exchanges (each step keeps half the heads), so the lanes of a
//      row end with one head's total each.  Shapes with one work-group per
//      CU read the three kinds of rows as one block-aligned stream instead.
//      T^ rows and the first V rows this thread contracts later are loaded at
//      the end of the pass, so their latency overlaps step 2.
//   2. per head (one wave): c = max lg, f = max s, fh = e^{s - f}; running-max
//      update for the evicted key (NystromHead::far_insert): r_i, e_i, Z^ and
//      m_max written back; u = fh . M; c_all = max(c, f + m_max); gain =
//      u e^{f + m_max - c_all}; far_den = gain . Z^; aggregate rectifier; near
//      weights p = e^{lg - shift} and the joint denominator.
//   3. column pass, one float4 column chunk per lane: T^ <- T^ r + e v_e written
//      back and contracted with gain in the same pass; V rows contracted with p.
//   4. reduce the row lanes (lane swaps within a wave, LDS across waves), one
//      division per output, counters.
// HBM traffic: each group's state read once and its modified part (one ring
// row, T^, Z^, m_max, counters) written once.
//
// Work-group size: 256 threads when the launch has many groups (several
// work-groups per CU hide each other's latency), 512 when it has few.
// A launch covers the groups of a GroupMap: the whole handle, or one layer of
// every sequence; inputs and outputs are indexed by the launch's own index.
#include <atomic>

#include "o1_internal.h"

namespace o1 {
namespace {

constexpr int kMaxDynLds = 32 * 1024;  // near logits: hpk * (sink + w) doubles

template <int D, int DV, int HPK, int MM, int NT>
struct DecodeShape {
    static constexpr int NW = NT / 64;                                 // waves
    static constexpr int CH = D / 4;                                   // float4 per key row
    static constexpr int LPR_WANT = HPK <= 2 ? 8 : (HPK <= 4 ? 16 : 32);
    static constexpr int LPR = LPR_WANT < CH ? LPR_WANT : CH;          // lanes per row
    static constexpr int CPL = CH / LPR;                               // float4 per lane per row
    static constexpr int RPW = 64 / LPR;                               // rows per wave per pass
    static constexpr int RPB = RPW * NW;                               // rows per block per pass
    static constexpr int UNR = CPL >= 4 ? 2 : (CPL == 2 ? 4 : 8);      // rows per lane in flight
    static constexpr int VCH = DV / 4;                                 // float4 per value row
    static constexpr int RL = NT / VCH;                                // row lanes, column pass
    static constexpr int RLW = 64 / VCH;                               // row lanes per wave
    static constexpr int TPT = (MM + RL - 1) / RL;                     // T^ rows per lane per head
    static constexpr bool STAGE_M = HPK * MM * MM <= 2048;             // M staged in LDS
    static constexpr bool PRE_T = HPK * TPT <= (NT == 256 ? 8 : 32);   // T^ prefetched in registers
    static constexpr int VPRE = NT == 256 ? (HPK <= 2 ? 8 : 4) : 8;    // V rows prefetched per lane
    static constexpr int VU = HPK <= 2 ? 9 : 8;                        // V rows per lane per batch
    static constexpr int MB = NT == 256 ? 16 : 32;                     // M rows in flight (unstaged M)
    static constexpr bool NTL = NT == 256;                             // streaming accesses (large grids)
    // One work-group per CU and registers to spare: the row pass runs as one
    // stream over every row it reads, two batches per round trip, with the
    // queries in f64 registers.
    static constexpr bool STREAM_ROWS = NT == 512 && HPK * D >= 512;
    // at least three waves per SIMD on large grids (at most 168 VGPRs)
    static constexpr int MIN_WAVES = NT == 256 ? 3 : 2;
    // heads per LDS round of the final reduction (one work-group per CU: room for all)
    static constexpr int RED_CAP = (STREAM_ROWS ? 65536 : 16384) / (NW * DV * 8);
    static constexpr int RED_H = HPK < RED_CAP ? HPK : RED_CAP;
    static_assert(D % (4 * LPR) == 0, "key width must split evenly over the row lanes");
    static_assert(HPK <= LPR, "the head reduction needs at least hpk lanes per row");
    static_assert(64 % VCH == 0, "value rows must tile a wave");
    static_assert(CH <= 64 && VCH <= 64, "rows wider than 256 floats are not compiled");
    static_assert(RED_H >= 1 && HPK % RED_H == 0, "heads must split into reduction rounds");
};

template <int D, int DV, int HPK, int MM, int NT>
__global__ __launch_bounds__(NT, (DecodeShape<D, DV, HPK, MM, NT>::MIN_WAVES)) void decode_kernel(DevState s, DecodeIO io)
{
    using C = DecodeShape<D, DV, HPK, MM, NT>;
    const int ci = blockIdx.x;            // call index: inputs and outputs
    const int g = io.map.state(ci);       // state group
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = s.sink, R = s.R, m = s.m;
    const double scale = (double)s.scale;
    const double NEG_INF = -__builtin_inf();

    __shared__ float4 q_s[HPK][C::CH];
    __shared__ float4 kn_s[C::CH], ke_s[C::CH];
    __shared__ float4 vn_s[C::VCH], ve_s[C::VCH];
    __shared__ float mo_s[HPK][MM];                // running max before this step
    __shared__ double zo_s[HPK][MM];               // Z^ before this step
    __shared__ float mu_s[C::STAGE_M ? HPK * MM * MM : 1];
    __shared__ double land_s[HPK][MM];             // landmark logits
    __shared__ double lf_s[HPK][MM];               // far-insert logits
    __shared__ double r_s[HPK][MM];                // T^ rescale factor per landmark
    __shared__ double e_s[HPK][MM];                // weight of the evicted key per landmark
    __shared__ double gain_s[HPK][MM];             // far mixing gains (0 when dropped)
    __shared__ double fh_s[C::STAGE_M ? HPK : 1][MM];  // landmark weights e^{s - f} (0 past m)
    __shared__ double den_s[HPK];
    __shared__ double red_s[C::NW][C::RED_H * DV];
    extern __shared__ double lg_s[];               // [HPK][R] near logits, then weights

    const size_t gh0 = (size_t)g * HPK;  // first head of this group
    const int e = s.win_head[g];
    const int slot_row = S + e;

    float4 *nk = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * R * C::CH;
    float4 *nv = reinterpret_cast<float4 *>(s.near_v) + (size_t)g * R * C::VCH;

    // ---- 0. prologue: small loads staged into LDS ---------------------------
    {
        const float4 *qg = reinterpret_cast<const float4 *>(io.q) + (size_t)ci * HPK * C::CH;
        for (int i = tid; i < HPK * C::CH; i += NT) (&q_s[0][0])[i] = qg[i];
        if (tid < C::CH) {
            kn_s[tid] = reinterpret_cast<const float4 *>(io.k)[(size_t)ci * C::CH + tid];
            ke_s[tid] = nk[(size_t)slot_row * C::CH + tid];
        }
        if (tid >= 128 && tid < 128 + C::VCH) {
            const int c = tid - 128;
            vn_s[c] = reinterpret_cast<const float4 *>(io.v)[(size_t)ci * C::VCH + c];
            ve_s[c] = nv[(size_t)slot_row * C::VCH + c];
        }
        for (int i = tid; i < HPK * m; i += NT) {
            const int h = i / m, a = i - h * m;
            mo_s[h][a] = s.m_max[gh0 * m + i];
            zo_s[h][a] = s.z_hat[gh0 * m + i];
        }
        if constexpr (C::STAGE_M) {
            const float *mu = s.mu + gh0 * (size_t)m * m;
            for (int i = tid; i < HPK * m * m; i += NT) mu_s[i] = mu[i];
        }
    }
    __syncthreads();
    if (tid < C::CH) nk[(size_t)slot_row * C::CH + tid] = kn_s[tid];
    if (tid >= 128 && tid < 128 + C::VCH) nv[(size_t)slot_row * C::VCH + tid - 128] = vn_s[tid - 128];

    // ---- 1. row-dot pass ----------------------------------------------------
    // Loads are unconditional (row indices clamped into range, results of
    // out-of-range rows discarded) so each batch issues back to back.
    const int cc = tid % C::VCH, rl = tid / C::VCH;  // column-pass mapping
    float4 tpre[C::PRE_T ? HPK : 1][C::PRE_T ? C::TPT : 1];
    float4 vpre[C::VPRE];
    {
        const int sub = lane % C::LPR, rsub = lane / C::LPR;
        constexpr int HSTRIDE = C::LPR / HPK;  // lanes per head after the head reduction
        const int my_head = sub / HSTRIDE;
        const bool writer = (sub % HSTRIDE) == 0;
        const float4 *kt = reinterpret_cast<const float4 *>(s.k_tilde) + (size_t)g * m * C::CH;
        const int NA = R + m;  // near rows, then landmark rows
        if constexpr (C::STREAM_ROWS) {
            // One row space in which each kind of row starts on a block row, so
            // the source of every load and the work on it are uniform across
            // the wave: [0, RP) near keys (R used), [RP, Q0) key landmarks (m
            // used), [Q0, NTOT) query landmarks (far-insert logits against the
            // evicted key).  Unused rows load a clamped row and are discarded.
            const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
            const int NQ = HPK * m;
            const int RP = (R + C::RPB - 1) / C::RPB * C::RPB;
            const int Q0 = (RP + m + C::RPB - 1) / C::RPB * C::RPB;
            const int NTOT = Q0 + NQ;
            constexpr int BR = C::UNR * C::RPB;  // rows per batch
            const int NB = (NTOT + BR - 1) / BR;
            const int r0 = wave * C::RPW + rsub;
            // this lane's columns of every query and of the evicted key, in f64
            // registers for the whole pass (one work-group per CU leaves room)
            double qd[HPK][C::CPL][4], kd[C::CPL][4];
#pragma unroll
            for (int k = 0; k < C::CPL; ++k) {
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    const float4 t = q_s[h][sub + C::LPR * k];
                    qd[h][k][0] = t.x, qd[h][k][1] = t.y, qd[h][k][2] = t.z, qd[h][k][3] = t.w;
                }
                const float4 t = ke_s[sub + C::LPR * k];
                kd[k][0] = t.x, kd[k][1] = t.y, kd[k][2] = t.z, kd[k][3] = t.w;
            }
            auto dotd = [](const double (&a)[4], const float4 x) {
                double s = a[0] * (double)x.x;
                s = fma(a[1], (double)x.y, s);
                s = fma(a[2], (double)x.z, s);
                s = fma(a[3], (double)x.w, s);
                return s;
            };
            auto load = [&](float4 (&x)[C::UNR][C::CPL], int b) {
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int rb = b * BR + u * C::RPB;  // first row of the block row (wave-uniform)
                    const int r = rb + r0;
                    const float4 *row = rb < RP ? nk + (size_t)min(r, R - 1) * C::CH
                                        : rb < Q0 ? kt + (size_t)min(r - RP, m - 1) * C::CH
                                                  : qt + (size_t)min(r - Q0, NQ - 1) * C::CH;
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) x[u][k] = ld4<C::NTL>(row + sub + C::LPR * k);
                }
            };
            auto reduce = [&](float4 (&x)[C::UNR][C::CPL], int b) {
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int rb = b * BR + u * C::RPB;
                    const int r = rb + r0;
                    if (rb < Q0) {
                        if (rb < RP && r == slot_row) {  // the ring slot already holds the new key
#pragma unroll
                            for (int k = 0; k < C::CPL; ++k) x[u][k] = kn_s[sub + C::LPR * k];
                        }
                        double part[HPK];
#pragma unroll
                        for (int h = 0; h < HPK; ++h) {
                            double acc = 0.0;
#pragma unroll
                            for (int k = 0; k < C::CPL; ++k) acc += dotd(qd[h][k], x[u][k]);
                            part[h] = acc;
                        }
                        const double tot = head_reduce<C::LPR, HPK>(part, lane) * scale;
                        if (writer) {
                            if (rb < RP) {
                                if (r < R) lg_s[my_head * R + r] = tot;
                            } else if (r - RP < m) {
                                land_s[my_head][r - RP] = tot;
                            }
                        }
                    } else {
                        double acc = 0.0;
#pragma unroll
                        for (int k = 0; k < C::CPL; ++k) acc += dotd(kd[k], x[u][k]);
                        acc = group_sum<C::LPR>(acc);
                        const int rq = r - Q0;
                        if (sub == 0 && rq < NQ) lf_s[rq / m][rq % m] = acc * scale;
                    }
                }
            };
            // two batches per round trip; no load stays in flight across the
            // loop's back edge, where the compiler's wait counting turns
            // conservative
            float4 xa[C::UNR][C::CPL], xb[C::UNR][C::CPL];
            for (int b = 0; b < NB; b += 2) {
                load(xa, b);
                if (b + 1 < NB) load(xb, b + 1);
                reduce(xa, b);
                if (b + 1 < NB) reduce(xb, b + 1);
            }
        } else {
            for (int base = wave * C::RPW; base < NA; base += C::UNR * C::RPB) {
                float4 x[C::UNR][C::CPL];
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int r = min(base + u * C::RPB + rsub, NA - 1);
                    const float4 *row = (r < R) ? nk + (size_t)r * C::CH : kt + (size_t)(r - R) * C::CH;
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) x[u][k] = ld4<C::NTL>(row + sub + C::LPR * k);
                }
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int r = base + u * C::RPB + rsub;
                    if (r == slot_row) {  // the ring slot already holds the new key
#pragma unroll
                        for (int k = 0; k < C::CPL; ++k) x[u][k] = kn_s[sub + C::LPR * k];
                    }
                    double part[HPK];
#pragma unroll
                    for (int h = 0; h < HPK; ++h) {
                        // keep q in LDS: re-read per row instead of pinning it in registers
                        asm volatile("" ::: "memory");
                        double acc = 0.0;
#pragma unroll
                        for (int k = 0; k < C::CPL; ++k) acc += dot4(q_s[h][sub + C::LPR * k], x[u][k]);
                        part[h] = acc;
                    }
                    const double tot = head_reduce<C::LPR, HPK>(part, lane) * scale;
                    if (writer) {
                        if (r < R) lg_s[my_head * R + r] = tot;
                        else if (r < NA) land_s[my_head][r - R] = tot;
                    }
                }
            }

            // far-insert logits of the evicted key against every query landmark
            float4 kr[C::CPL];
#pragma unroll
            for (int k = 0; k < C::CPL; ++k) kr[k] = ke_s[sub + C::LPR * k];
            const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
            const int NQ = HPK * m;
            for (int base = wave * C::RPW; base < NQ; base += C::UNR * C::RPB) {
                float4 x[C::UNR][C::CPL];
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int r = min(base + u * C::RPB + rsub, NQ - 1);
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) x[u][k] = ld4<C::NTL>(qt + (size_t)r * C::CH + sub + C::LPR * k);
                }
#pragma unroll
                for (int u = 0; u < C::UNR; ++u) {
                    const int r = base + u * C::RPB + rsub;
                    double acc = 0.0;
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) acc += dot4(x[u][k], kr[k]);
                    acc = group_sum<C::LPR>(acc);
                    if (sub == 0 && r < NQ) lf_s[r / m][r % m] = acc * scale;
                }
            }
        }

        // prefetch: this thread's T^ rows and its first V rows
        if constexpr (C::PRE_T) {
            const float4 *th = reinterpret_cast<const float4 *>(s.t_hat) + gh0 * m * C::VCH;
#pragma unroll
            for (int h = 0; h < HPK; ++h)
#pragma unroll
                for (int j = 0; j < C::TPT; ++j) {
                    const int b = min(rl + j * C::RL, m - 1);
                    tpre[h][j] = ld4<C::NTL>(th + ((size_t)h * m + b) * C::VCH + cc);
                }
        }
#pragma unroll
        for (int j = 0; j < C::VPRE; ++j) {
            const int r = min(rl + j * C::RL, R - 1);
            vpre[j] = ld4<C::NTL>(nv + (size_t)r * C::VCH + cc);
        }
    }
    __syncthreads();

    // ---- 2. per-head landmark work and near weights (one wave per head) ----
    for (int h = wave; h < HPK; h += C::NW) {
        double c = NEG_INF;
        for (int r = lane; r < R; r += 64) c = fmax(c, lg_s[h * R + r]);
        c = wave_max(c);

        const bool act = lane < m;
        const double sa = act ? land_s[h][lane] : NEG_INF;
        const double f = wave_max(sa);
        const double fh = act ? exp(sa - f) : 0.0;

        // NystromHead::far_insert for landmark i = lane: strict ">" growth of
        // the running max; T^ and Z^ stay at scale e^{-m_max} with m_max kept
        // as the f32 value actually stored.
        const size_t hi = (gh0 + h) * m + lane;
        double mn = NEG_INF, zn = 0.0;
        if (act) {
            const double l = lf_s[h][lane];
            const float mo = mo_s[h][lane];
            float mnf = mo;
            double r = 1.0;
            if (l > (double)mo) {
                mnf = (float)l;
                r = exp((double)mo - (double)mnf);
            }
            mn = (double)mnf;
            const double ee = exp(l - mn);
            zn = zo_s[h][lane] * r + ee;
            s.m_max[hi] = mnf;
            s.z_hat[hi] = zn;
            r_s[h][lane] = r;
            e_s[h][lane] = ee;
        }

        // u_b = sum_a fh_a M[a][b]  (lane = b)
        double u = 0.0;
        if constexpr (C::STAGE_M) {
            // fh goes through LDS (zero past m): the loop runs over the
            // compile-time bound MM with broadcast reads and clamped rows of
            // the staged M, without branches or cross-lane shuffles.
            if (lane < MM) fh_s[h][lane] = fh;
            __builtin_amdgcn_wave_barrier();
            const float *mu = mu_s + (size_t)h * m * m;
            const int col = act ? lane : 0;
#pragma unroll 8
            for (int a = 0; a < MM; ++a) u = fma(fh_s[h][a], (double)mu[min(a, m - 1) * m + col], u);
            if (!act) u = 0.0;
        } else {
            // M from global memory, MB rows per lane in flight
            const float *mu = s.mu + (gh0 + h) * (size_t)m * m;
            const int col = act ? lane : 0;
            for (int a0 = 0; a0 < m; a0 += C::MB) {
                float mv[C::MB];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) mv[j] = mu[(size_t)min(a0 + j, m - 1) * m + col];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) {
                    const double fa = lane_value(fh, (a0 + j) & 63);
                    if (a0 + j < m && act) u = fma(fa, (double)mv[j], u);
                }
            }
        }
        if (s.rect == 1) u = fmax(u, 0.0);  // O1Rect::Fm

        const double call = fmax(c, wave_max(act ? f + mn : NEG_INF));
        const double gain = act ? u * exp(f + mn - call) : 0.0;
        const double far_den = wave_sum(gain * zn);
        const bool keep = far_den >= 0.0;  // aggregate rectifier (0 keeps)
        if (act) gain_s[h][lane] = keep ? gain : 0.0;
        const double shift = keep ? call : c;  // dropped far field: near-only shift

        double acc = 0.0;
        for (int r = lane; r < R; r += 64) {
            const double p = exp(lg_s[h * R + r] - shift);
            lg_s[h * R + r] = p;
            acc += p;
        }
        acc = wave_sum(acc);
        if (lane == 0) den_s[h] = (keep ? far_den : 0.0) + acc;
    }
    __syncthreads();

    // ---- 3. column pass: T^ update + far contraction, V contraction --------
    double acc[HPK][4];
#pragma unroll
    for (int h = 0; h < HPK; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.0;
    {
        float4 *th = reinterpret_cast<float4 *>(s.t_hat) + gh0 * m * C::VCH;
        const float4 vev = ve_s[cc];
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
#pragma unroll
            for (int j = 0; j < C::TPT; ++j) {
                const int b = rl + j * C::RL;
                if (b >= m) break;
                const size_t idx = ((size_t)h * m + b) * C::VCH + cc;
                float4 t;
                if constexpr (C::PRE_T) t = tpre[h][j];
                else t = ld4<C::NTL>(th + idx);
                const double rb = r_s[h][b], eb = e_s[h][b], gb = gain_s[h][b];
                const double t0 = fma((double)t.x, rb, eb * (double)vev.x);
                const double t1 = fma((double)t.y, rb, eb * (double)vev.y);
                const double t2 = fma((double)t.z, rb, eb * (double)vev.z);
                const double t3 = fma((double)t.w, rb, eb * (double)vev.w);
                st4<C::NTL>(th + idx, make_float4((float)t0, (float)t1, (float)t2, (float)t3));
                acc[h][0] = fma(gb, t0, acc[h][0]);
                acc[h][1] = fma(gb, t1, acc[h][1]);
                acc[h][2] = fma(gb, t2, acc[h][2]);
                acc[h][3] = fma(gb, t3, acc[h][3]);
            }
        }
    }
    {
        // V rows r = rl + j * RL: the first VPRE were prefetched before step 2
#pragma unroll
        for (int j = 0; j < C::VPRE; ++j) {
            const int r = rl + j * C::RL;
            if (r >= R) break;
            const float4 x = (r == slot_row) ? vn_s[cc] : vpre[j];
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                const double p = lg_s[h * R + r];
                acc[h][0] = fma(p, (double)x.x, acc[h][0]);
                acc[h][1] = fma(p, (double)x.y, acc[h][1]);
                acc[h][2] = fma(p, (double)x.z, acc[h][2]);
                acc[h][3] = fma(p, (double)x.w, acc[h][3]);
            }
        }
        for (int r0 = rl + C::VPRE * C::RL; r0 < R; r0 += C::VU * C::RL) {
            float4 x[C::VU];
#pragma unroll
            for (int j = 0; j < C::VU; ++j) x[j] = ld4<C::NTL>(nv + (size_t)min(r0 + j * C::RL, R - 1) * C::VCH + cc);
#pragma unroll
            for (int j = 0; j < C::VU; ++j) {
                const int r = r0 + j * C::RL;
                if (r >= R) break;
                if (r == slot_row) x[j] = vn_s[cc];
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    const double p = lg_s[h * R + r];
                    acc[h][0] = fma(p, (double)x[j].x, acc[h][0]);
                    acc[h][1] = fma(p, (double)x[j].y, acc[h][1]);
                    acc[h][2] = fma(p, (double)x[j].z, acc[h][2]);
                    acc[h][3] = fma(p, (double)x[j].w, acc[h][3]);
                }
            }
        }
    }

    // ---- 4. reduce row lanes, joint division, counters ---------------------
    // within a wave: the RLW row lanes sit VCH lanes apart
#pragma unroll
    for (int h = 0; h < HPK; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[h][c] = sum_high_lanes<C::VCH>(acc[h][c]);
    float4 *outp = reinterpret_cast<float4 *>(io.out) + (size_t)ci * HPK * C::VCH;
#pragma unroll
    for (int h0 = 0; h0 < HPK; h0 += C::RED_H) {
        if (lane < C::VCH) {
#pragma unroll
            for (int hh = 0; hh < C::RED_H; ++hh) {
                double *dst = &red_s[wave][hh * DV + cc * 4];
                dst[0] = acc[h0 + hh][0];
                dst[1] = acc[h0 + hh][1];
                dst[2] = acc[h0 + hh][2];
                dst[3] = acc[h0 + hh][3];
            }
        }
        __syncthreads();
        if (tid < C::RED_H * C::VCH) {
            const int hh = tid / C::VCH, c4 = tid - hh * C::VCH;
            double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
#pragma unroll
            for (int j = 0; j < C::NW; ++j) {
                const double *src = &red_s[j][hh * DV + c4 * 4];
                o0 += src[0];
                o1 += src[1];
                o2 += src[2];
                o3 += src[3];
            }
            const double den = fmax(den_s[h0 + hh], kDenEps);
            outp[(size_t)(h0 + hh) * C::VCH + c4] =
                make_float4((float)(o0 / den), (float)(o1 / den), (float)(o2 / den), (float)(o3 / den));
        }
        if (h0 + C::RED_H < HPK) __syncthreads();
    }
    if (tid == 0) s.win_head[g] = (e + 1 == s.w) ? 0 : e + 1;
    if (tid < HPK) s.far_len[gh0 + tid] += 1;
}

template <int D, int DV, int HPK, int MM, int NT>
hipError_t launch_shape(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    // Static LDS of the wide shapes plus the near logits can pass 64 KB; raise
    // the kernel's dynamic limit once per device (function attributes are per
    // device; an unsupported size fails the launch).
    static std::atomic<uint64_t> done{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = dev < 64 ? 1ull << dev : 0;
    if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_kernel<D, DV, HPK, MM, NT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
        if (err != hipSuccess) return err;
        done.fetch_or(bit, std::memory_order_release);
    }
    const size_t dyn = sizeof(double) * (size_t)HPK * s.R;
    hipLaunchKernelGGL((decode_kernel<D, DV, HPK, MM, NT>), dim3(io.map.count), dim3(NT), dyn, stream, s, io);
    return hipGetLastError();
}

// Few groups per launch leave CUs with a single work-group, whose latency is
// then exposed: use 512 threads per group there.
constexpr int kSmallGrid = 1024;

template <int D, int DV, int HPK, int MM>
hipError_t launch_nt(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    if (io.map.count < kSmallGrid) return launch_shape<D, DV, HPK, MM, 512>(s, io, stream);
    return launch_shape<D, DV, HPK, MM, 256>(s, io, stream);
}

template <int D, int DV, int HPK>
hipError_t launch_m(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    if (s.m <= 32) return launch_nt<D, DV, HPK, 32>(s, io, stream);
    return launch_nt<D, DV, HPK, kMaxLandmarks>(s, io, stream);
}

template <int D, int DV>
hipError_t launch_hpk(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    switch (s.hpk) {
    case 1: return launch_m<D, DV, 1>(s, io, stream);
    case 2: return launch_m<D, DV, 2>(s, io, stream);
    case 4: return launch_m<D, DV, 4>(s, io, stream);
    case 8: return launch_m<D, DV, 8>(s, io, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_supported(int d, int dv, int hpk, int m, int R)
{
    if (!(d == dv && (d == 64 || d == 128))) return false;
    if (!(hpk == 1 || hpk == 2 || hpk == 4 || hpk == 8)) return false;
    if (m < 4 || m > kMaxLandmarks) return false;
    if (R < 1 || R > 1024) return false;
    // dynamic LDS for the near logits stays within 32 KB
    return (size_t)hpk * R * sizeof(double) <= (size_t)kMaxDynLds;
}

hipError_t launch_decode(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    if (!decode_supported(s.d, s.dv, s.hpk, s.m, s.R)) return hipErrorInvalidValue;
    if (s.d == 64) return launch_hpk<64, 64>(s, io, stream);
    return launch_hpk<128, 128>(s, io, stream);
}

}  // namespace o1
