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
//      running max, its value at the last fold and Z^, (small shapes) each
//      head's mixing matrix M, and the held evictions (kPend): with P =
//      far_len mod kPend, the value rows and logits of slots j < P, whose
//      logits become weights e^{l - m_max} against the running max before
//      this step.  Every load is issued before any is stored (one round
//      trip).  Then row sink+e is overwritten by the new k/v (advance); the
//      evicted value row joins the held set (slot P) unless this step folds.
//   1. row-dot pass, f64 accumulation, each row split over LPR lanes and UNR
//      rows per lane in flight:
//        near logits  lg[h][r] = q_h . k_r * scale       (sink + w rows, all heads)
//        landmark     s[h][a]  = q_h . k~_a * scale      (m rows, all heads)
//        far insert   l[h][i]  = q~_{h,i} . k_e * scale  (hpk * m rows)
//      The hpk partial dots of a row are reduced over the row's lanes by
//      halving exchanges (each step keeps half the heads), so the lanes of a
//      row end with one head's total each.  Shapes with one work-group per
//      CU read the three kinds of rows as one block-aligned stream instead,
//      and with eight heads take the dots on f64 MFMA (16-row tiles times the
//      queries and the evicted key as columns).
//      T^ rows and the first V rows this thread contracts later are loaded at
//      the end of the pass, so their latency overlaps step 2.
//   2. per head (one wave): c = max lg, f = max s, fh = e^{s - f}; running-max
//      update for the evicted key (NystromHead::far_insert): Z^ and m_max
//      written back, the held weights moved to the new max, the eviction's
//      logit stored in slot P (or, on a fold, m_ref = m_max); u = fh . M;
//      c_all = max(c, f + m_max); gain = u e^{f + m_max - c_all}; far_den =
//      gain . Z^; aggregate rectifier; near weights p = e^{lg - shift} and the
//      joint denominator.  Between folds each held row and the eviction's row
//      get one coefficient sum_i gain_i w_ij (a wave sum per row).
//   3. column pass, one float4 column chunk per lane: the far numerator
//      gain . T^ with T^ = e^{m_ref - m_max} t_hat + sum_j w_j v_j -- between
//      folds t_hat is only read and the held rows are contracted with their
//      coefficients; on a fold t_hat is rebuilt at the new max and written
//      back -- then the V rows contracted with p.
//   4. reduce the row lanes (lane swaps within a wave, LDS across waves), one
//      division per output, counters.
// HBM traffic: each group's state read once; the ring row, Z^, m_max, the held
// slot and the counters written every step, t_hat once per kPend steps.
//
// Work-group size: 256 threads when the launch has many groups (several
// work-groups per CU hide each other's latency), 512 when it has few or when
// the shape's LDS allows only one work-group per CU anyway (hpk * m >= 512).
// State loads and stores are nontemporal when the state is streamed from HBM.
// A launch covers the groups of a GroupMap: the whole handle, or one layer of
// every sequence; inputs and outputs are indexed by the launch's own index.
#include <atomic>
#include <type_traits>

#include "o1_internal.h"

namespace o1 {
namespace {

constexpr int kMaxDynLds = 32 * 1024;  // near logits: hpk * (sink + w) doubles

template <int D, int DV, int HPK, int MM, int NT, bool STREAM>
struct DecodeShape {
    static constexpr int NW = NT / 64;                                 // waves
    static constexpr int CH = D / 4;                                   // float4 per key row
    static constexpr int LPR_WANT = HPK <= 2 ? 8 : (HPK <= 4 ? 16 : 32);
    static constexpr int LPR = pow2_divisor(LPR_WANT, CH);             // lanes per row
    static constexpr int CPL = CH / LPR;                               // float4 per lane per row
    static constexpr int RPW = 64 / LPR;                               // rows per wave per pass
    static constexpr int RPB = RPW * NW;                               // rows per block per pass
    static constexpr int UNR = CPL >= 8 ? 1 : (CPL >= 4 ? 2 : (CPL == 3 ? 3 : (CPL == 2 ? 4 : 8)));  // rows per lane in flight
    static constexpr int UNR_NEAR = (NT == 512 && CPL >= 4 && CPL < 8) ? 3 : UNR;  // near + landmark rows (row pass)
    static constexpr int VCH = DV / 4;                                 // float4 per value row
    static constexpr int VCP = pow2_ceil(VCH);                         // lanes per value row (VCH used)
    static constexpr int RL = NT / VCP;                                // row lanes, column pass
    static constexpr int RLW = 64 / VCP;                               // row lanes per wave
    static constexpr int TPT = (MM + RL - 1) / RL;                     // T^ rows per lane per head
    static constexpr bool STAGE_M = HPK * MM * MM <= 2048;             // M staged in LDS
    static constexpr bool PRE_T = HPK * TPT <= (NT == 256 ? 8 : (DV > 128 ? 16 : 32));  // T^ prefetched in registers
    // otherwise heads per block of T^ loads in flight (at most 8 rows per lane)
    static constexpr int TB = TPT >= 8 ? 1 : (8 / TPT < HPK ? 8 / TPT : HPK);
    // V rows prefetched per lane (6 where 8 would spill at 256 VGPRs; 9 at 512
    // threads covers a 128-key window plus 4 sinks, so no V batch follows)
    static constexpr int VPRE = NT == 256 ? (HPK <= 2 ? 8 : 4) : (HPK * MM >= 512 ? 6 : 9);
    static constexpr int VU = HPK <= 2 ? 9 : 8;                        // V rows per lane per batch
    static constexpr int MB = NT == 256 ? 16 : 32;                     // M rows in flight (unstaged M)
    static constexpr bool NTL = STREAM;                                // nontemporal state accesses
    // One work-group per CU and registers to spare: the row pass runs as one
    // stream over every row it reads, two batches per round trip, with the
    // queries in f64 registers.
    static constexpr bool STREAM_ROWS = NT == 512 && HPK * D >= 512 && (CH & (CH - 1)) == 0 && HPK * CPL <= 8;
    // eight heads: the row pass takes its dots on f64 MFMA (rows x [queries,
    // evicted key]) instead of per-lane dots and head reductions, in the
    // streamed form's launches and in 256-thread ones (rows of at most 128
    // floats: a tile's operands stay in registers)
    static constexpr bool MFMA_ROWS = HPK == 8 && D % 16 == 0 && D <= 128 && (STREAM_ROWS || NT == 256);
    static constexpr int HL = (HPK * kPend * MM + NT - 1) / NT;       // held logits per thread
    // per-head phase: two heads per wave, one per half-wave (m <= 32)
    static constexpr bool PAIR_HEADS = NT == 256 && HPK == 2 * NW && MM == 32;
    // at least three waves per SIMD on large grids (at most 168 VGPRs)
    static constexpr int MIN_WAVES = NT == 256 ? 3 : 2;
    // heads per LDS round of the final reduction (one work-group per CU: room for all)
    static constexpr int RED_CAP = pow2_floor((STREAM_ROWS ? 65536 : 16384) / (NW * DV * 8));
    static constexpr int RED_H = HPK < RED_CAP ? HPK : RED_CAP;
    // the final reduction's buffer also holds the held weights (steps 0-3)
    static constexpr int RED_N = NW * RED_H * DV, WF_N = HPK * kPend * MM;
    static constexpr int SHARE_N = RED_N > WF_N ? RED_N : WF_N;
    static_assert(D % (4 * LPR) == 0, "key width must split evenly over the row lanes");
    static_assert(HPK <= LPR, "the head reduction needs at least hpk lanes per row");
    static_assert(64 % VCP == 0, "value rows must tile a wave");
    static_assert(CH <= 64 && VCH <= 64, "rows wider than 256 floats are not compiled");
    static_assert(RED_H >= 1 && HPK % RED_H == 0, "heads must split into reduction rounds");
    static_assert(RL >= kPend, "each held value row needs a row lane of its own");
    static_assert((kPend - 1) * VCH <= NT, "one held value float4 per thread");
    static_assert(HPK * MM <= NT && 128 + VCH <= NT,
                  "the prologue loads at most one element of each kind per thread (but queries and the fold's keys)");
};

template <int D, int DV, int HPK, int MM, int NT, bool STREAM, bool PART>
__global__ __launch_bounds__(NT, (DecodeShape<D, DV, HPK, MM, NT, STREAM>::MIN_WAVES)) void decode_kernel(DevState s, DecodeIO io)
{
    using C = DecodeShape<D, DV, HPK, MM, NT, STREAM>;
    const int ci = blockIdx.x;            // call index: inputs and outputs
    const int g = io.map.state(ci);       // state group
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = s.sink, R = s.R, m = s.m;
    // query heads of the group: HPK is the compiled count (a power of two), H
    // the group's own.  With PART (HPK / 2 < H < HPK) heads H .. HPK-1 are
    // placeholders: zero queries, no state read or written, no output; their
    // LDS slots hold values nothing stores.  Without it H is the compile-time
    // HPK (full groups keep every index a constant).
    const int H = PART ? io.hb : HPK;
    // the group's own head count, the stride of every per-head array, and the
    // first head of this launch's block
    const int HG = s.hpk, h0 = io.h0;
    // 256-thread launches skip the placeholder heads' column sums and
    // reductions (uniform branches on H); 512-thread ones would spill for it
    constexpr bool SKIP_PH = PART && NT == 256;
    const double scale = (double)s.scale;
    const double NEG_INF = -__builtin_inf();

    __shared__ float4 q_s[HPK][C::CH];
    __shared__ float4 kn_s[C::CH], ke_s[C::CH];
    __shared__ float4 vn_s[C::VCH], ve_s[C::VCH];
    __shared__ float4 hv_s[kPend - 1][C::VCH];     // value rows of the held evictions (slots j < P)
    __shared__ float4 kb_s[kPend][C::CH];          // fold with ring logits: the keys that arrived since the last fold
    __shared__ float mo_s[HPK][MM];                // running max before this step
    __shared__ float mr_s[HPK][MM];                // running max at the last fold (scale of t_hat)
    __shared__ double zo_s[HPK][MM];               // Z^ before this step
    __shared__ float mu_s[C::STAGE_M ? HPK * MM * MM : 1];
    __shared__ double land_s[HPK][MM];             // landmark logits
    __shared__ double lf_s[HPK][MM];               // far-insert logits
    __shared__ double r_s[HPK][MM];                // fold: stored t_hat -> new max, per landmark
    __shared__ double cj_s[HPK][kPend];            // held slot j (and this eviction, slot P): sum_i gain_i w_ij
    __shared__ double gain_s[HPK][MM];             // far mixing gains (0 when dropped), times r between folds
    __shared__ double fh_s[C::STAGE_M || C::PAIR_HEADS ? HPK : 1][MM];  // landmark weights e^{s - f} (0 past m)
    __shared__ double den_s[HPK];
    // held logits, then their weights at the new max, [HPK][kPend][MM] (steps 0-3);
    // then the reduction across waves, [NW][RED_H * DV] (step 4)
    __shared__ double share_s[C::SHARE_N];
    auto wf_s = reinterpret_cast<double (*)[kPend][MM]>(share_s);
    auto red_s = reinterpret_cast<double (*)[C::RED_H * DV]>(share_s);
    extern __shared__ double lg_s[];               // [HPK][R] near logits, then weights

    const size_t gh0 = (size_t)g * HG + h0;  // first head of this block
    const int e = min(max(s.win_head[g], 0), s.w - 1);  // (in range unless written out of range)
    const int slot_row = S + e;
    // evictions held apart from t_hat before this step, and whether this
    // step's eviction completes the set (then all are folded into t_hat)
    const int P = (int)((uint64_t)s.far_len[gh0] % kPend);
    const bool fold = P == kPend - 1;
    // far-insert logits kept per ring slot (w >= kPend): the evicted key's are
    // read, and a fold computes those of the keys that arrived since the last
    // one (slots e, e-1, ..., e-kPend+1), so q~ is read once per kPend steps
    const bool ring = s.ring_l != nullptr;
    const int w = s.w;

    float4 *nk = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * R * C::CH;
    float4 *nv = reinterpret_cast<float4 *>(s.near_v) + (size_t)g * R * C::VCH;

    // 512-thread launches without the streamed row pass: the row pass's first
    // batch of near and landmark rows is issued with the prologue's loads (the
    // rows do not depend on them; the ring slot the prologue overwrites is
    // replaced by the new key when its dot is taken)
    constexpr bool HOIST = NT == 512 && !C::STREAM_ROWS;
    const float4 *kt_rows = reinterpret_cast<const float4 *>(s.k_tilde) + (size_t)g * m * C::CH;
    float4 xh[HOIST ? C::UNR_NEAR : 1][C::CPL];

    // ---- 0. prologue: small loads staged into LDS ---------------------------
    {
        // held evictions, slots j < P: loads issued first, stored at the end
        float4 hvr = make_float4(0.f, 0.f, 0.f, 0.f);
        const bool hv_mine = tid < P * C::VCH;
        if (hv_mine) hvr = ld4<C::NTL>(reinterpret_cast<const float4 *>(s.pend_v) + (size_t)g * kPend * C::VCH + tid);
        double hlr[C::HL];
        const int nl = H * kPend * m;  // [h][j][a] block of this group
#pragma unroll
        for (int u = 0; u < C::HL; ++u) {
            const int i = tid + u * NT;
            hlr[u] = 0.0;
            if (i < nl && (i / m) % kPend < P) hlr[u] = s.pend_l[gh0 * kPend * m + i];
        }
        const float4 *qg = reinterpret_cast<const float4 *>(io.q) + ((size_t)ci * HG + h0) * C::CH;
        // every load is issued before any is stored, so the prologue costs
        // one round trip (each thread has at most one element of most kinds;
        // a few of M, and of the queries and the fold's keys at wide rows)
        const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
        // the block's queries, QP float4 per thread (placeholder heads: zero)
        constexpr int QP = (HPK * C::CH + NT - 1) / NT;
        const bool k_mine = tid < C::CH;
        const bool v_mine = tid >= 128 && tid < 128 + C::VCH, st_mine = tid < H * m;
        // on a fold with ring logits, the keys that arrived since the last
        // fold (ring slots e-1 .. e-kPend+1): KBP float4 per thread
        constexpr int KBP = ((kPend - 1) * C::CH + NT - 1) / NT;
        const bool kb_fold = ring && fold;
        float4 kbv[KBP];
        float4 qv[QP], kin = z4, kev = z4, vin = z4, vev = z4;
#pragma unroll
        for (int u = 0; u < QP; ++u) {
            const int i = tid + u * NT;
            qv[u] = z4;
            if (i < H * C::CH) qv[u] = qg[i];
        }
        if (k_mine) {
            kin = reinterpret_cast<const float4 *>(io.k)[(size_t)ci * C::CH + tid];
            if (!ring) kev = nk[(size_t)slot_row * C::CH + tid];
        }
#pragma unroll
        for (int u = 0; u < KBP; ++u) {
            const int i = tid + u * NT, j = 1 + i / C::CH, c = i - (j - 1) * C::CH;
            kbv[u] = z4;
            if (kb_fold && i < (kPend - 1) * C::CH) kbv[u] = nk[(size_t)(S + (e - j + w) % w) * C::CH + c];
        }
        if (v_mine) {
            vin = reinterpret_cast<const float4 *>(io.v)[(size_t)ci * C::VCH + tid - 128];
            vev = nv[(size_t)slot_row * C::VCH + tid - 128];
        }
        float mo = 0.f, mr = 0.f;
        double zo = 0.0, lr = 0.0;
        if (st_mine) {
            mo = s.m_max[gh0 * m + tid];
            mr = s.m_ref[gh0 * m + tid];
            zo = s.z_hat[gh0 * m + tid];
            if (ring) lr = s.ring_l[(((size_t)g * w + e) * HG + h0) * m + tid];
        }
        constexpr int MUP = C::STAGE_M ? (HPK * MM * MM + NT - 1) / NT : 1;
        float muv[MUP];
        if constexpr (C::STAGE_M) {
            const float *mu = s.mu + gh0 * (size_t)m * m;
#pragma unroll
            for (int u = 0; u < MUP; ++u) {
                const int i = tid + u * NT;
                muv[u] = i < H * m * m ? mu[i] : 0.f;
            }
        }
        // after the prologue's own loads, so that its stores below wait for
        // those alone (loads complete in order)
        if constexpr (HOIST) {
            const int sub = lane % C::LPR, rsub = lane / C::LPR, NA = R + m;
#pragma unroll
            for (int u = 0; u < C::UNR_NEAR; ++u) {
                const int r = min(wave * C::RPW + u * C::RPB + rsub, NA - 1);
                const float4 *row = (r < R) ? nk + (size_t)r * C::CH : kt_rows + (size_t)(r - R) * C::CH;
#pragma unroll
                for (int k = 0; k < C::CPL; ++k) xh[u][k] = ld4<C::NTL>(row + sub + C::LPR * k);
            }
        }
#pragma unroll
        for (int u = 0; u < QP; ++u)
            if (tid + u * NT < HPK * C::CH) (&q_s[0][0])[tid + u * NT] = qv[u];
        if (k_mine) {
            kn_s[tid] = kin;
            if (!ring) ke_s[tid] = kev;
            else if (fold) kb_s[0][tid] = kin;
        }
#pragma unroll
        for (int u = 0; u < KBP; ++u) {
            const int i = tid + u * NT, j = 1 + i / C::CH, c = i - (j - 1) * C::CH;
            if (kb_fold && i < (kPend - 1) * C::CH) kb_s[j][c] = kbv[u];
        }
        if (v_mine) {
            vn_s[tid - 128] = vin;
            ve_s[tid - 128] = vev;
        }
        if (st_mine) {
            const int h = tid / m, a = tid - h * m;
            mo_s[h][a] = mo;
            mr_s[h][a] = mr;
            zo_s[h][a] = zo;
            if (ring) lf_s[h][a] = lr;
        }
        if constexpr (C::STAGE_M) {
#pragma unroll
            for (int u = 0; u < MUP; ++u) {
                const int i = tid + u * NT;
                if (i < H * m * m) mu_s[i] = muv[u];
            }
        }
        if (hv_mine) (&hv_s[0][0])[tid] = hvr;
        __syncthreads();
        // held weights at the running max before this step (at most 1 up to
        // the f32 rounding of the stored max, which covers every held logit);
        // step 2 rescales them to the new max
#pragma unroll
        for (int u = 0; u < C::HL; ++u) {
            const int i = tid + u * NT;
            const int hj = i / m, a = i - hj * m;
            if (i < nl && hj % kPend < P)
                wf_s[hj / kPend][hj % kPend][a] = exp(hlr[u] - (double)mo_s[hj / kPend][a]);
        }
    }
    // the group's shared writes (the last head block's launch; every launch
    // reads the ring slot's old row in its prologue and uses the new key and
    // value from LDS for that slot)
    if (io.shared) {
        if (tid < C::CH) nk[(size_t)slot_row * C::CH + tid] = kn_s[tid];
        if (tid >= 128 && tid < 128 + C::VCH) {
            nv[(size_t)slot_row * C::VCH + tid - 128] = vn_s[tid - 128];
            // the evicted value row joins the held set (slot P) unless this step folds
            if (!fold) reinterpret_cast<float4 *>(s.pend_v)[((size_t)g * kPend + P) * C::VCH + tid - 128] = ve_s[tid - 128];
        }
    }

    // ---- 1. row-dot pass ----------------------------------------------------
    // Loads are unconditional (row indices clamped into range, results of
    // out-of-range rows discarded) so each batch issues back to back.
    // column-pass mapping: column lane cp of row lane rl; lanes past a row's VCH
    // columns (VCH not a power of two) repeat its last column and store nothing
    const int cp = tid % C::VCP, rl = tid / C::VCP, cc = min(cp, C::VCH - 1);
    float4 tpre[C::PRE_T ? HPK : 1][C::PRE_T ? C::TPT : 1];
    float4 vpre[C::VPRE];
    {
        const int sub = lane % C::LPR, rsub = lane / C::LPR;
        constexpr int HSTRIDE = C::LPR / HPK;  // lanes per head after the head reduction
        const int my_head = sub / HSTRIDE;
        const bool writer = (sub % HSTRIDE) == 0;
        const float4 *kt = reinterpret_cast<const float4 *>(s.k_tilde) + (size_t)g * m * C::CH;
        const int NA = R + m;  // near rows, then landmark rows
        if constexpr (C::MFMA_ROWS) {
            // Row space [0, R) near keys, [R, R + m) key landmarks, [R + m, NR)
            // query landmarks (far-insert logits of the evicted key; none with
            // ring logits), in 16-row tiles, times B = [q_0 .. q_7, k_e, 0 ..]:
            // D[row][j] is the dot of the row with head j's query (j < 8) or
            // with the evicted key (j = 8).  Operand layout (wave64): A[i][k] in
            // lane i + 16 k, B[k][j] in lane j + 16 k; f64 D[i][j] in lane
            // j + 16 (i % 4), element i / 4.  In MFMA step (jj, c), k-lane kk
            // stands for component 16 jj + 4 kk + c of A and B alike, so a lane's
            // operands of one row are the D/16 float4 at 4 jj + kk.  Rows past NR
            // load a clamped row and are discarded.
            constexpr int NJ = D / 16;
            using d4v = __attribute__((ext_vector_type(4))) double;
            const int li = lane & 15, lk = lane >> 4;
            const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
            const int NQ = ring ? 0 : H * m, NR = R + m + NQ, NTILE = (NR + 15) / 16;
            float4 bq[NJ];  // column li of B: head li's query, or the evicted key
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) {
                const float4 q = q_s[min(li, HPK - 1)][4 * jj + lk], k = ke_s[4 * jj + lk];
                bq[jj] = li < HPK ? q : (li == HPK && !ring ? k : make_float4(0.f, 0.f, 0.f, 0.f));
            }
            auto loadA = [&](float4 (&x)[NJ], int t) {
                const int r = min(16 * t + li, NR - 1);
                const float4 *row = r < R ? nk + (size_t)r * C::CH
                                  : r < R + m ? kt + (size_t)(r - R) * C::CH
                                              : qt + (size_t)(r - R - m) * C::CH;
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) x[jj] = ld4<C::NTL>(row + 4 * jj + lk);
            };
            auto mma = [&](float4 (&x)[NJ], int t) {
                if (16 * t + li == slot_row) {  // the ring slot already holds the new key
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) x[jj] = kn_s[4 * jj + lk];
                }
                d4v acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].x, (double)bq[jj].x, acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].y, (double)bq[jj].y, acc2, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].z, (double)bq[jj].z, acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].w, (double)bq[jj].w, acc2, 0, 0, 0);
                }
                acc += acc2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * t + 4 * e + lk;  // D[4 e + lk][li]
                    const double v = acc[e] * scale;
                    if (li < HPK) {
                        if (row < R) lg_s[li * R + row] = v;
                        else if (row < R + m) land_s[li][row - R] = v;
                    } else if (li == HPK && row >= R + m && row < NR) {
                        const int rq = row - R - m;
                        lf_s[rq / m][rq % m] = v;
                    }
                }
            };
            // two tiles per round trip
            float4 xa[NJ], xb[NJ];
            for (int t = wave; t < NTILE; t += 2 * C::NW) {
                loadA(xa, t);
                if (t + C::NW < NTILE) loadA(xb, t + C::NW);
                mma(xa, t);
                if (t + C::NW < NTILE) mma(xb, t + C::NW);
            }
        } else if constexpr (C::STREAM_ROWS) {
            // One row space in which each kind of row starts on a block row, so
            // the source of every load and the work on it are uniform across
            // the wave: [0, RP) near keys (R used), [RP, Q0) key landmarks (m
            // used), [Q0, NTOT) query landmarks (far-insert logits of the
            // evicted key; none with ring logits).  Unused rows load a clamped
            // row and are discarded.
            const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
            const int NQ = H * m;
            const int RP = (R + C::RPB - 1) / C::RPB * C::RPB;
            const int Q0 = (RP + m + C::RPB - 1) / C::RPB * C::RPB;
            const int NTOT = Q0 + (ring ? 0 : NQ);
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
                const float4 t = ring ? make_float4(0.f, 0.f, 0.f, 0.f) : ke_s[sub + C::LPR * k];
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
                    } else if (rb >= NTOT) {
                        // past the row space (the last batch's tail): nothing
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
            for (int base = wave * C::RPW; base < NA; base += C::UNR_NEAR * C::RPB) {
                float4 x[C::UNR_NEAR][C::CPL];
                if (HOIST && base == wave * C::RPW) {
#pragma unroll
                    for (int u = 0; u < C::UNR_NEAR; ++u)
#pragma unroll
                        for (int k = 0; k < C::CPL; ++k) x[u][k] = xh[HOIST ? u : 0][k];
                } else {
#pragma unroll
                    for (int u = 0; u < C::UNR_NEAR; ++u) {
                        const int r = min(base + u * C::RPB + rsub, NA - 1);
                        const float4 *row = (r < R) ? nk + (size_t)r * C::CH : kt + (size_t)(r - R) * C::CH;
#pragma unroll
                        for (int k = 0; k < C::CPL; ++k) x[u][k] = ld4<C::NTL>(row + sub + C::LPR * k);
                    }
                }
#pragma unroll
                for (int u = 0; u < C::UNR_NEAR; ++u) {
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

            // far-insert logits against every query landmark: of the evicted key
            // (no ring logits), or, on a fold with ring logits, of the keys
            // that arrived since the last fold (stored per ring slot)
            const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
            const int NQ = H * m;
            if (!ring) {
                float4 kr[C::CPL];
#pragma unroll
                for (int k = 0; k < C::CPL; ++k) kr[k] = ke_s[sub + C::LPR * k];
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
            } else if (fold) {
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
#pragma unroll 1
                        for (int j = 0; j < kPend; ++j) {
                            double acc = 0.0;
#pragma unroll
                            for (int k = 0; k < C::CPL; ++k) acc += dot4(x[u][k], kb_s[j][sub + C::LPR * k]);
                            acc = group_sum<C::LPR>(acc);
                            if (sub == 0 && r < NQ)
                                s.ring_l[(((size_t)g * w + (e - j + w) % w) * HG + h0) * m + r] = acc * scale;
                        }
                    }
                }
            }
        }

        // on a fold with ring logits, shapes with the streamed or MFMA row pass
        // (many heads): the far-insert logits of the kPend latest keys against every
        // query landmark, a [hpk m x D] x [D x kPend] product on f64 MFMA in
        // 16-row tiles (the other shapes take them in the row pass, whose rows
        // span few lanes).  A = q~ rows, read through the cache; B = the keys,
        // from LDS, zero for j >= kPend.  The reduction index is permuted so the
        // four k-lanes of a row read 64 contiguous bytes per load: in MFMA step
        // (jj, c), k-lane kk stands for component 16 jj + 4 kk + c of A and B.
        // (D[i][j] in lane j + 16 (i mod 4), element i / 4)
        if ((C::STREAM_ROWS || C::MFMA_ROWS) && ring && fold) {
            const int NQ = H * m;
            const int li = lane & 15, lk = lane >> 4;
            const float4 *qt4 = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH + lk;
            const float4 *kb4 = &kb_s[min(li, kPend - 1)][lk];
            const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int t = wave; t < (NQ + 15) / 16; t += C::NW) {
                const float4 *qa = qt4 + (size_t)min(16 * t + li, NQ - 1) * C::CH;
                __attribute__((ext_vector_type(4))) double acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int jj = 0; jj < D / 16; ++jj) {
                    const float4 a = qa[4 * jj];
                    float4 b = z4;
                    if (li < kPend) b = kb4[4 * jj];
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.x, (double)b.x, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.y, (double)b.y, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.z, (double)b.z, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)a.w, (double)b.w, acc, 0, 0, 0);
                }
                if (li < kPend) {
                    double *dst = s.ring_l + (((size_t)g * w + (e - li + w) % w) * HG + h0) * m;
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int r = 16 * t + 4 * r4 + lk;
                        if (r < NQ) dst[r] = acc[r4] * scale;
                    }
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
                    tpre[h][j] = ld4<C::NTL>(th + ((size_t)min(h, H - 1) * m + b) * C::VCH + cc);
                }
        }
#pragma unroll
        for (int j = 0; j < C::VPRE; ++j) {
            const int r = min(rl + j * C::RL, R - 1);
            vpre[j] = ld4<C::NTL>(nv + (size_t)r * C::VCH + cc);
        }
    }
    __syncthreads();

    // ---- 2. per-head landmark work and near weights ------------------------
    // One head per wave (W = 64 lanes), or, in 256-thread launches of eight
    // heads with m <= 32, one head per half-wave (W = 32: heads 2 wave and
    // 2 wave + 1 side by side, so each instruction serves two heads).  Lane la
    // of the head's W owns landmark la; reductions run over the W lanes.
    auto per_head = [&](auto width, int h, int la, bool live) {
        constexpr int W = decltype(width)::value;
        auto wmax = [](double x) {
            if constexpr (W == 64) return wave_max(x);
            else return group_max<16>(swap_max<16>(x));
        };
        auto wsum = [](double x) { return group_sum<W>(x); };
        const bool act = la < m;
        const bool stores = act && live;  // placeholder halves compute, but store nothing
        const size_t hi = (gh0 + h) * m + la;
        double c = NEG_INF;
        for (int r = la; r < R; r += W) c = fmax(c, lg_s[h * R + r]);
        c = wmax(c);

        const double sa = act ? land_s[h][la] : NEG_INF;
        const double f = wmax(sa);
        const double fh = act ? exp(sa - f) : 0.0;

        // NystromHead::far_insert for landmark i = la: strict ">" growth of
        // the running max; Z^ stays at scale e^{-m_max} with m_max kept as the
        // f32 value actually stored.  T^ gets the same update through the held
        // set: this eviction's weight is ee at the new max.
        double mn = NEG_INF, zn = 0.0;
        if (act) {
            const double lnew = lf_s[h][la];
            const float mo = mo_s[h][la];
            float mnf = mo;
            double r = 1.0;
            if (lnew > (double)mo) {
                mnf = (float)lnew;
                r = exp((double)mo - (double)mnf);
            }
            mn = (double)mnf;
            const double ee = exp(lnew - mn);
            zn = zo_s[h][la] * r + ee;
            if (live) {
                s.m_max[hi] = mnf;
                s.z_hat[hi] = zn;
                // T^_i = rf_i t_hat_i + sum_{j<P} w_ij v_j + ee_i v_e at the new
                // max: the held weights move from the old max to the new one,
                // and this eviction's weight takes slot P (on a fold, slot
                // kPend - 1)
                r_s[h][la] = exp((double)mr_s[h][la] - mn);
                for (int j = 0; j < P; ++j) wf_s[h][j][la] *= r;
                wf_s[h][fold ? kPend - 1 : P][la] = ee;
                if (fold) s.m_ref[hi] = mnf;
                else s.pend_l[(gh0 + h) * kPend * (size_t)m + (size_t)P * m + la] = lnew;
            }
        }

        // u_b = sum_a fh_a M[a][b]  (la = b)
        double u = 0.0;
        if constexpr (C::STAGE_M) {
            // fh goes through LDS (zero past m): the loop runs over the
            // compile-time bound MM with broadcast reads and clamped rows of
            // the staged M, without branches or cross-lane shuffles.
            if (la < MM) fh_s[h][la] = fh;
            __builtin_amdgcn_wave_barrier();
            const float *mu = mu_s + (size_t)h * m * m;
            const int col = act ? la : 0;
#pragma unroll 8
            for (int a = 0; a < MM; ++a) u = fma(fh_s[h][a], (double)mu[min(a, m - 1) * m + col], u);
            if (!act) u = 0.0;
        } else {
            // M from global memory, MB rows per lane in flight; fh_a from
            // lane a (one head per wave) or through LDS (two per wave)
            const float *mu = s.mu + (gh0 + (W == 32 ? min(h, H - 1) : h)) * (size_t)m * m;
            const int col = act ? la : 0;
            if constexpr (W == 32) {
                fh_s[h][la] = fh;
                __builtin_amdgcn_wave_barrier();
            }
            for (int a0 = 0; a0 < m; a0 += C::MB) {
                float mv[C::MB];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) mv[j] = mu[(size_t)min(a0 + j, m - 1) * m + col];
#pragma unroll
                for (int j = 0; j < C::MB; ++j) {
                    double fa;
                    if constexpr (W == 64) fa = lane_value(fh, (a0 + j) & 63);
                    else fa = fh_s[h][(a0 + j) & 31];
                    if (a0 + j < m && act) u = fma(fa, (double)mv[j], u);
                }
            }
        }
        if (s.rect == 1) u = fmax(u, 0.0);  // O1Rect::Fm

        const double call = fmax(c, wmax(act ? f + mn : NEG_INF));
        const double gain = act ? u * exp(f + mn - call) : 0.0;
        const double far_den = wsum(gain * zn);
        const bool keep = far_den >= 0.0;  // aggregate rectifier (0 keeps)
        const double gk = keep ? gain : 0.0;
        const double shift = keep ? call : c;  // dropped far field: near-only shift

        if (fold) {
            // the column pass rebuilds t_hat at the new max
            if (stores) gain_s[h][la] = gk;
        } else {
            // t_hat stays as stored: its gains carry rf, and each held row and
            // this eviction's row (slot P) gets one coefficient sum_i gain_i w_ij
            if (stores) gain_s[h][la] = gk * r_s[h][la];
            for (int j = 0; j <= P; ++j) {
                const double cj = wsum(act ? gk * wf_s[h][j][la] : 0.0);
                if (la == 0 && live) cj_s[h][j] = cj;
            }
        }

        double acc = 0.0;
        for (int r = la; r < R; r += W) {
            const double p = exp(lg_s[h * R + r] - shift);
            if (live) lg_s[h * R + r] = p;
            acc += p;
        }
        acc = wsum(acc);
        if (la == 0 && live) den_s[h] = (keep ? far_den : 0.0) + acc;
    };
    if constexpr (C::PAIR_HEADS) {
        const int h = 2 * wave + (lane >> 5);
        if (2 * wave < H) per_head(std::integral_constant<int, 32>{}, h, lane & 31, h < H);
    } else {
        for (int h = wave; h < H; h += C::NW) per_head(std::integral_constant<int, 64>{}, h, lane, true);
    }
    __syncthreads();

    // ---- 3. column pass: far contraction (t_hat rebuilt on a fold), V contraction
    double acc[HPK][4];
#pragma unroll
    for (int h = 0; h < HPK; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.0;
    {
        float4 *th = reinterpret_cast<float4 *>(s.t_hat) + gh0 * m * C::VCH;
        if (fold) {
            // t_hat <- r t_hat + sum_j w_j v_j over the held rows and this
            // eviction's, written back once for kPend steps
            auto fold_row = [&](int h, int b, float4 t) {
                const size_t idx = ((size_t)min(h, H - 1) * m + b) * C::VCH + cc;
                const double rb = r_s[h][b], gb = gain_s[h][b];
                double t0 = (double)t.x * rb, t1 = (double)t.y * rb;
                double t2 = (double)t.z * rb, t3 = (double)t.w * rb;
                // held row k + 1 loaded while row k is added in
                double wk = wf_s[h][0][b];
                float4 x = hv_s[0][cc];
#pragma unroll 1
                for (int k = 1; k < kPend; ++k) {
                    const double wn = wf_s[h][k][b];
                    const float4 xn = k < kPend - 1 ? hv_s[k][cc] : ve_s[cc];
                    t0 = fma(wk, (double)x.x, t0);
                    t1 = fma(wk, (double)x.y, t1);
                    t2 = fma(wk, (double)x.z, t2);
                    t3 = fma(wk, (double)x.w, t3);
                    wk = wn;
                    x = xn;
                }
                t0 = fma(wk, (double)x.x, t0);
                t1 = fma(wk, (double)x.y, t1);
                t2 = fma(wk, (double)x.z, t2);
                t3 = fma(wk, (double)x.w, t3);
                if (h < H && cp < C::VCH)
                    st4<C::NTL>(th + idx, make_float4((float)t0, (float)t1, (float)t2, (float)t3));
                acc[h][0] = fma(gb, t0, acc[h][0]);
                acc[h][1] = fma(gb, t1, acc[h][1]);
                acc[h][2] = fma(gb, t2, acc[h][2]);
                acc[h][3] = fma(gb, t3, acc[h][3]);
            };
            if constexpr (C::PRE_T) {
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
#pragma unroll
                    for (int j = 0; j < C::TPT; ++j) {
                        const int b = rl + j * C::RL;
                        if (b >= m) break;
                        fold_row(h, b, tpre[h][j]);
                    }
                }
            } else {
                // T^ rows in blocks of TB heads, each block's loads issued
                // before its rows are folded (rows past m load row m - 1 and
                // are skipped)
#pragma unroll
                for (int h0 = 0; h0 < HPK; h0 += C::TB) {
                    if (SKIP_PH && h0 >= H) break;
                    float4 t[C::TB][C::TPT];
#pragma unroll
                    for (int hh = 0; hh < C::TB; ++hh)
#pragma unroll
                        for (int j = 0; j < C::TPT; ++j)
                            t[hh][j] = ld4<C::NTL>(th + ((size_t)min(h0 + hh, H - 1) * m + min(rl + j * C::RL, m - 1)) * C::VCH + cc);
#pragma unroll
                    for (int hh = 0; hh < C::TB; ++hh) {
                        const int h = h0 + hh;
                        if (SKIP_PH && h >= H) break;
#pragma unroll
                        for (int j = 0; j < C::TPT; ++j) {
                            const int b = rl + j * C::RL;
                            if (b < m) fold_row(h, b, t[hh][j]);
                        }
                        // as in the step without a fold: one block's rows live at a time
                        asm volatile("" : "+v"(acc[h][0]), "+v"(acc[h][1]), "+v"(acc[h][2]), "+v"(acc[h][3])::"memory");
                    }
                }
            }
        } else {
            if constexpr (C::PRE_T) {
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
#pragma unroll
                    for (int j = 0; j < C::TPT; ++j) {
                        const int b = rl + j * C::RL;
                        if (b >= m) break;
                        const float4 t = tpre[h][j];
                        const double gb = gain_s[h][b];
                        acc[h][0] = fma(gb, (double)t.x, acc[h][0]);
                        acc[h][1] = fma(gb, (double)t.y, acc[h][1]);
                        acc[h][2] = fma(gb, (double)t.z, acc[h][2]);
                        acc[h][3] = fma(gb, (double)t.w, acc[h][3]);
                    }
                }
            } else {
                // T^ rows in blocks of TB heads, every load of a block issued
                // before its rows are added in (rows past m load row m - 1 and
                // weigh 0), so a block costs one round trip
#pragma unroll
                for (int h0 = 0; h0 < HPK; h0 += C::TB) {
                    if (SKIP_PH && h0 >= H) break;  // placeholder heads only
                    float4 t[C::TB][C::TPT];
#pragma unroll
                    for (int hh = 0; hh < C::TB; ++hh)
#pragma unroll
                        for (int j = 0; j < C::TPT; ++j)
                            t[hh][j] = ld4<C::NTL>(th + ((size_t)min(h0 + hh, H - 1) * m + min(rl + j * C::RL, m - 1)) * C::VCH + cc);
#pragma unroll
                    for (int hh = 0; hh < C::TB; ++hh) {
                        const int h = h0 + hh;
                        if (SKIP_PH && h >= H) break;
#pragma unroll
                        for (int j = 0; j < C::TPT; ++j) {
                            const int b = rl + j * C::RL;
                            const double gb = b < m ? gain_s[h][b] : 0.0;
                            acc[h][0] = fma(gb, (double)t[hh][j].x, acc[h][0]);
                            acc[h][1] = fma(gb, (double)t[hh][j].y, acc[h][1]);
                            acc[h][2] = fma(gb, (double)t[hh][j].z, acc[h][2]);
                            acc[h][3] = fma(gb, (double)t[hh][j].w, acc[h][3]);
                        }
                        // the block's sums are complete here and the next block's
                        // loads stay behind them: one block's rows live at a time
                        asm volatile("" : "+v"(acc[h][0]), "+v"(acc[h][1]), "+v"(acc[h][2]), "+v"(acc[h][3])::"memory");
                    }
                }
            }
            // row lane j < P: held slot j; row lane P: this eviction
            if (rl <= P) {
                const float4 x = rl < P ? hv_s[rl][cc] : ve_s[cc];
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    if (SKIP_PH && h >= H) break;
                    const double cj = cj_s[h][rl];
                    acc[h][0] = fma(cj, (double)x.x, acc[h][0]);
                    acc[h][1] = fma(cj, (double)x.y, acc[h][1]);
                    acc[h][2] = fma(cj, (double)x.z, acc[h][2]);
                    acc[h][3] = fma(cj, (double)x.w, acc[h][3]);
                }
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
                if (SKIP_PH && h >= H) break;  // placeholder heads: nothing to add
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
                    if (SKIP_PH && h >= H) break;
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
    if (fold) __syncthreads();  // every wave is done with the fold weights
    // within a wave: the RLW row lanes sit VCP lanes apart
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        if (SKIP_PH && h >= H) break;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[h][c] = sum_high_lanes<C::VCP>(acc[h][c]);
    }
    float4 *outp = reinterpret_cast<float4 *>(io.out) + ((size_t)ci * HG + h0) * C::VCH;
#pragma unroll
    for (int h0 = 0; h0 < HPK; h0 += C::RED_H) {
        if (SKIP_PH && h0 >= H) break;  // uniform: every thread leaves together
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
        if (tid < C::RED_H * C::VCH && h0 + tid / C::VCH < H) {
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
    if (tid == 0 && io.shared) s.win_head[g] = (e + 1 == s.w) ? 0 : e + 1;
    if (tid < H) s.far_len[gh0 + tid] += 1;
}

template <int D, int DV, int HPK, int MM, int NT, bool STREAM, bool PART>
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
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(&decode_kernel<D, DV, HPK, MM, NT, STREAM, PART>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
        if (err != hipSuccess) return err;
        done.fetch_or(bit, std::memory_order_release);
    }
    const size_t dyn = sizeof(double) * (size_t)HPK * s.R;
    hipLaunchKernelGGL((decode_kernel<D, DV, HPK, MM, NT, STREAM, PART>), dim3(io.map.count), dim3(NT), dyn, stream, s, io);
    return hipGetLastError();
}

// Few groups per launch leave CUs with a single work-group, whose latency is
// then exposed: use 512 threads per group there.  Shapes with hpk * m >= 512
// (e.g. 8 heads, 64 landmarks) need so much LDS that 256-thread work-groups
// would also run one per CU, so they take 512 threads at every grid size.
// State accesses are nontemporal when the handle's state is larger than the
// Infinity Cache (it is then streamed from HBM at every step, also one layer at
// a time), and cached when it fits there; 256-thread launches (>= 1024 groups)
// always stream.
constexpr int kSmallGrid = 1024;

template <int D, int DV, int HPK, int MM, bool PART>
hipError_t launch_nt(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    const bool big = s.stream_state != 0;
    // (value rows wider than 128 floats: 512 threads keep a row lane per held slot)
    if constexpr (HPK * MM < 512 && DV <= 128) {
        if (io.map.count >= kSmallGrid) return launch_shape<D, DV, HPK, MM, 256, true, PART>(s, io, stream);
    }
    if (big) return launch_shape<D, DV, HPK, MM, 512, true, PART>(s, io, stream);
    return launch_shape<D, DV, HPK, MM, 512, false, PART>(s, io, stream);
}

template <int D, int DV, int HPK, bool PART = false>
hipError_t launch_m(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    if (s.m <= 32) return launch_nt<D, DV, HPK, 32, PART>(s, io, stream);
    return launch_nt<D, DV, HPK, kMaxLandmarks, PART>(s, io, stream);
}

template <int D, int DV>
hipError_t launch_hpk(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    // a block of hb heads runs the kernel compiled for the next power of two;
    // its variant for partial blocks takes the head count at run time
    switch (io.hb) {
    case 1: return launch_m<D, DV, 1>(s, io, stream);
    case 2: return launch_m<D, DV, 2>(s, io, stream);
    case 3: return launch_m<D, DV, 4, true>(s, io, stream);
    case 4: return launch_m<D, DV, 4>(s, io, stream);
    case 5:
    case 6:
    case 7:
        if constexpr (block_heads(D) >= 8) return launch_m<D, DV, 8, true>(s, io, stream);
        return hipErrorInvalidValue;
    case 8:
        if constexpr (block_heads(D) >= 8) return launch_m<D, DV, 8>(s, io, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

// One work-group per (group, head): T^ with the held evictions folded in, at
// the current running max, written to dst; with `reset` the held set is then
// emptied (m_ref = m_max, every slot's logits -inf).  Not on the decode path:
// state reads and writes use it.
__global__ __launch_bounds__(256) void fold_kernel(DevState s, float *dst, int reset)
{
    const int g = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int m = s.m, VCH = s.dv / 4;
    const size_t gh = (size_t)g * s.hpk + h;
    const int P = (int)((uint64_t)s.far_len[gh] % kPend);
    __shared__ double w_s[kPend][kMaxLandmarks], r_s[kMaxLandmarks];
    for (int a = tid; a < m; a += 256) {
        const double mx = (double)s.m_max[gh * m + a];
        r_s[a] = exp((double)s.m_ref[gh * m + a] - mx);
        for (int j = 0; j < kPend; ++j)
            w_s[j][a] = j < P ? exp(s.pend_l[(gh * kPend + j) * m + a] - mx) : 0.0;
    }
    __syncthreads();
    const float4 *th = reinterpret_cast<const float4 *>(s.t_hat) + gh * m * VCH;
    const float4 *pv = reinterpret_cast<const float4 *>(s.pend_v) + (size_t)g * kPend * VCH;
    float4 *out = reinterpret_cast<float4 *>(dst) + gh * m * VCH;
    for (int i = tid; i < m * VCH; i += 256) {
        const int a = i / VCH, c = i - a * VCH;
        const float4 t = th[i];
        const double rb = r_s[a];
        double t0 = (double)t.x * rb, t1 = (double)t.y * rb, t2 = (double)t.z * rb, t3 = (double)t.w * rb;
        for (int j = 0; j < P; ++j) {
            const float4 v = pv[(size_t)j * VCH + c];
            const double wj = w_s[j][a];
            t0 = fma(wj, (double)v.x, t0);
            t1 = fma(wj, (double)v.y, t1);
            t2 = fma(wj, (double)v.z, t2);
            t3 = fma(wj, (double)v.w, t3);
        }
        out[i] = make_float4((float)t0, (float)t1, (float)t2, (float)t3);
    }
    if (!reset) return;
    for (int a = tid; a < m; a += 256) {
        s.m_ref[gh * m + a] = s.m_max[gh * m + a];
        for (int j = 0; j < kPend; ++j) s.pend_l[(gh * kPend + j) * m + a] = -__builtin_inf();
    }
}

}  // namespace

hipError_t launch_fold(const DevState &s, float *dst, bool reset, hipStream_t stream)
{
    if (s.m < 1 || s.m > kMaxLandmarks || s.dv % 4 || (reset && dst != s.t_hat)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fold_kernel, dim3(s.G, s.hpk), dim3(256), 0, stream, s, dst, reset ? 1 : 0);
    return hipGetLastError();
}

bool decode_supported(int d, int dv, int hpk, int m, int R)
{
    if (!widths_compiled(d, dv)) return false;
    if (hpk < 1 || hpk > kMaxHeads) return false;
    if (m < 4 || m > kMaxLandmarks) return false;
    if (R < 1 || R > 4096) return false;
    // dynamic LDS for the near logits of the compiled head count (hpk rounded
    // up to a power of two) stays within 32 KB: sink + w up to 4096 at one
    // head per block, 2048 at two, 1024 at four, 512 at eight
    const int bh = block_heads(d);
    const int hb = hpk < bh ? hpk : bh;  // heads of the largest block
    const int hc = hb <= 1 ? 1 : hb <= 2 ? 2 : hb <= 4 ? 4 : 8;
    return (size_t)hc * R * sizeof(double) <= (size_t)kMaxDynLds;
}

hipError_t launch_decode(const DevState &s, const DecodeIO &io_in, hipStream_t stream)
{
    if (!decode_supported(s.d, s.dv, s.hpk, s.m, s.R)) return hipErrorInvalidValue;
    // groups of more heads than a block holds (block_heads): one launch per block,
    // in order on the stream; the last makes the group's shared writes
    const int bh = block_heads(s.d);
    for (int h0 = 0; h0 < s.hpk; h0 += bh) {
        DecodeIO io = io_in;
        io.h0 = h0;
        io.hb = min(bh, s.hpk - h0);
        io.shared = h0 + bh >= s.hpk;
        hipError_t err;
        if (s.d == 64) err = launch_hpk<64, 64>(s, io, stream);
        else if (s.d == 96) err = launch_hpk<96, 96>(s, io, stream);
        else if (s.d == 256) err = launch_hpk<256, 256>(s, io, stream);
        else if (s.d == 192) err = launch_hpk<192, 128>(s, io, stream);
        else if (s.d == 80) err = launch_hpk<80, 80>(s, io, stream);
        else err = launch_hpk<128, 128>(s, io, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace o1
