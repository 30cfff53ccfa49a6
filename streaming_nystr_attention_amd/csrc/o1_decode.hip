// One decode step of streaming Nystrom attention for every group: the
// NystromState::step_group of the nystrom.rs source page (advance, then
// NystromHead::step per query head), batched as one work-group per group.
//
// Per work-group (256 threads = 4 wave64), in dependency order:
//   0. read the evicted ring slot e = win_head (row sink+e) and the new k/v into
//      LDS, then overwrite row sink+e with the new k/v (advance).  Nothing reads
//      that row from global memory afterwards.
//   1. row-dot pass, f64 accumulation, lanes split each row across LPR lanes:
//        near logits  lg[h][r] = q_h . k_r * scale       (sink + w rows, all heads)
//        landmark     s[h][a]  = q_h . k~_a * scale      (m rows, all heads)
//        far insert   l[h][i]  = q~_{h,i} . k_e * scale  (hpk * m rows)
//   2. per head (one wave): c = max lg, f = max s, fh = e^{s - f}; running-max
//      update of the evicted key (NystromHead::far_insert): r_i, e_i, Z^ and
//      m_max written back; u = fh . M; c_all = max(c, f + m_max); gain =
//      u e^{f + m_max - c_all}; far_den = gain . Z^; aggregate rectifier.
//   3. near weights p = e^{lg - shift} and the joint denominator.
//   4. column pass, one float4 column chunk per lane: T^ <- T^ r + e v_e written
//      back and contracted with gain in the same pass; V rows contracted with p.
//   5. reduce the row-lanes, one division per output, counters.
// The HBM stream is each group's state read once and its modified part (one
// ring row, T^, Z^, m_max, counters) written once.
#include "o1_internal.h"

namespace o1 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int D, int DV, int HPK>
struct DecodeShape {
    static constexpr int CH = D / 4;                                   // float4 per key row
    static constexpr int LPR_WANT = HPK <= 2 ? 8 : (HPK <= 4 ? 16 : 32);
    static constexpr int LPR = LPR_WANT < CH ? LPR_WANT : CH;          // lanes per row
    static constexpr int CPL = CH / LPR;                               // float4 per lane per row
    static constexpr int RPW = 64 / LPR;                               // rows per wave per pass
    static constexpr int RPB = RPW * kWaves;                           // rows per block per pass
    static constexpr int VCH = DV / 4;                                 // float4 per value row
    static constexpr int RL = kThreads / VCH;                          // row lanes, column pass
    static_assert(D % (4 * LPR) == 0, "key width must split evenly over the row lanes");
    static_assert(kThreads % VCH == 0, "value width must divide the block");
    static_assert(CH <= 64 && VCH <= 64, "rows wider than 256 floats are not compiled");
};

__device__ __forceinline__ double dot4(const float4 a, const float4 b)
{
    double s = (double)a.x * (double)b.x;
    s = fma((double)a.y, (double)b.y, s);
    s = fma((double)a.z, (double)b.z, s);
    s = fma((double)a.w, (double)b.w, s);
    return s;
}

template <int D, int DV, int HPK>
__global__ __launch_bounds__(kThreads) void decode_kernel(DevState s, DecodeIO io)
{
    using C = DecodeShape<D, DV, HPK>;
    const int g = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = s.sink, R = s.R, m = s.m;
    const double scale = (double)s.scale;
    const double NEG_INF = -__builtin_inf();

    __shared__ float4 q_s[HPK][C::CH];
    __shared__ float4 kn_s[C::CH], ke_s[C::CH];
    __shared__ float4 vn_s[C::VCH], ve_s[C::VCH];
    __shared__ double land_s[HPK][kMaxLandmarks];  // landmark logits
    __shared__ double lf_s[HPK][kMaxLandmarks];    // far-insert logits
    __shared__ double r_s[HPK][kMaxLandmarks];     // T^ rescale factor per landmark
    __shared__ double e_s[HPK][kMaxLandmarks];     // weight of the evicted key per landmark
    __shared__ double gain_s[HPK][kMaxLandmarks];  // far mixing gains (0 when dropped)
    __shared__ double shift_s[HPK], den_s[HPK];
    __shared__ double red_s[C::RL][DV];
    extern __shared__ double lg_s[];               // [HPK][R] near logits, then weights

    const size_t gh0 = (size_t)g * HPK;  // first head of this group
    const int e = s.win_head[g];
    const int slot_row = S + e;

    float4 *nk = reinterpret_cast<float4 *>(s.near_k) + (size_t)g * R * C::CH;
    float4 *nv = reinterpret_cast<float4 *>(s.near_v) + (size_t)g * R * C::VCH;

    // ---- 0. inputs and the evicted row into LDS; ring write -------------
    {
        const float4 *qg = reinterpret_cast<const float4 *>(io.q) + gh0 * C::CH;
        for (int i = tid; i < HPK * C::CH; i += kThreads) (&q_s[0][0])[i] = qg[i];
        if (tid < C::CH) {
            kn_s[tid] = reinterpret_cast<const float4 *>(io.k)[(size_t)g * C::CH + tid];
            ke_s[tid] = nk[(size_t)slot_row * C::CH + tid];
        }
        if (tid >= 128 && tid < 128 + C::VCH) {
            const int c = tid - 128;
            vn_s[c] = reinterpret_cast<const float4 *>(io.v)[(size_t)g * C::VCH + c];
            ve_s[c] = nv[(size_t)slot_row * C::VCH + c];
        }
    }
    __syncthreads();
    if (tid < C::CH) nk[(size_t)slot_row * C::CH + tid] = kn_s[tid];
    if (tid >= 128 && tid < 128 + C::VCH) nv[(size_t)slot_row * C::VCH + tid - 128] = vn_s[tid - 128];

    // ---- 1. row-dot pass --------------------------------------------------
    {
        const int sub = lane % C::LPR, rsub = lane / C::LPR;
        float4 qr[HPK][C::CPL];
#pragma unroll
        for (int h = 0; h < HPK; ++h)
#pragma unroll
            for (int k = 0; k < C::CPL; ++k) qr[h][k] = q_s[h][sub + C::LPR * k];

        const float4 *kt = reinterpret_cast<const float4 *>(s.k_tilde) + (size_t)g * m * C::CH;
        const int NA = R + m;  // near rows, then landmark rows
        for (int base = wave * C::RPW; base < NA; base += 2 * C::RPB) {
            float4 x[2][C::CPL];
            int rr[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = base + u * C::RPB + rsub;
                rr[u] = r;
#pragma unroll
                for (int k = 0; k < C::CPL; ++k) {
                    const int c = sub + C::LPR * k;
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (r < R) v = (r == slot_row) ? kn_s[c] : nk[(size_t)r * C::CH + c];
                    else if (r < NA) v = kt[(size_t)(r - R) * C::CH + c];
                    x[u][k] = v;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = rr[u];
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    double acc = 0.0;
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) acc += dot4(qr[h][k], x[u][k]);
                    acc = group_sum<C::LPR>(acc);
                    if (sub == 0) {
                        if (r < R) lg_s[h * R + r] = acc * scale;
                        else if (r < NA) land_s[h][r - R] = acc * scale;
                    }
                }
            }
        }

        // far-insert logits of the evicted key against every query landmark
        float4 kr[C::CPL];
#pragma unroll
        for (int k = 0; k < C::CPL; ++k) kr[k] = ke_s[sub + C::LPR * k];
        const float4 *qt = reinterpret_cast<const float4 *>(s.q_tilde) + gh0 * m * C::CH;
        const int NQ = HPK * m;
        for (int base = wave * C::RPW; base < NQ; base += 2 * C::RPB) {
            float4 x[2][C::CPL];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = base + u * C::RPB + rsub;
#pragma unroll
                for (int k = 0; k < C::CPL; ++k)
                    x[u][k] = (r < NQ) ? qt[(size_t)r * C::CH + sub + C::LPR * k]
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = base + u * C::RPB + rsub;
                double acc = 0.0;
#pragma unroll
                for (int k = 0; k < C::CPL; ++k) acc += dot4(x[u][k], kr[k]);
                acc = group_sum<C::LPR>(acc);
                if (sub == 0 && r < NQ) lf_s[r / m][r % m] = acc * scale;
            }
        }
    }
    __syncthreads();

    // ---- 2. per-head landmark work (one wave per head) --------------------
    for (int h = wave; h < HPK; h += kWaves) {
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
            const float mo = s.m_max[hi];
            float mnf = mo;
            double r = 1.0;
            if (l > (double)mo) {
                mnf = (float)l;
                r = exp((double)mo - (double)mnf);
            }
            mn = (double)mnf;
            const double ee = exp(l - mn);
            zn = s.z_hat[hi] * r + ee;
            s.m_max[hi] = mnf;
            s.z_hat[hi] = zn;
            r_s[h][lane] = r;
            e_s[h][lane] = ee;
        }

        // u_b = sum_a fh_a M[a][b]  (lane = b)
        const float *mu = s.mu + (gh0 + h) * (size_t)m * m;
        double u = 0.0;
        for (int a = 0; a < m; ++a) {
            const double fa = __shfl(fh, a, 64);
            if (act) u = fma(fa, (double)mu[(size_t)a * m + lane], u);
        }
        if (s.rect == 1) u = fmax(u, 0.0);  // O1Rect::Fm

        const double call = fmax(c, wave_max(act ? f + mn : NEG_INF));
        const double gain = act ? u * exp(f + mn - call) : 0.0;
        const double far_den = wave_sum(gain * zn);
        const bool keep = far_den >= 0.0;  // aggregate rectifier (0 keeps)
        if (act) gain_s[h][lane] = keep ? gain : 0.0;
        if (lane == 0) {
            shift_s[h] = keep ? call : c;  // dropped far field: near-only shift
            den_s[h] = keep ? far_den : 0.0;
        }
    }
    __syncthreads();

    // ---- 3. near weights and the joint denominator ------------------------
    for (int h = wave; h < HPK; h += kWaves) {
        const double sh = shift_s[h];
        double acc = 0.0;
        for (int r = lane; r < R; r += 64) {
            const double p = exp(lg_s[h * R + r] - sh);
            lg_s[h * R + r] = p;
            acc += p;
        }
        acc = wave_sum(acc);
        if (lane == 0) den_s[h] += acc;
    }
    __syncthreads();

    // ---- 4. column pass: T^ update + far contraction, V contraction -------
    const int cc = tid % C::VCH, rl = tid / C::VCH;
    double acc[HPK][4];
#pragma unroll
    for (int h = 0; h < HPK; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.0;
    {
        float4 *th = reinterpret_cast<float4 *>(s.t_hat) + gh0 * m * C::VCH;
        const float4 vev = ve_s[cc];
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
            for (int b = rl; b < m; b += C::RL) {
                const size_t idx = ((size_t)h * m + b) * C::VCH + cc;
                const float4 t = th[idx];
                const double rb = r_s[h][b], eb = e_s[h][b], gb = gain_s[h][b];
                const double t0 = fma((double)t.x, rb, eb * (double)vev.x);
                const double t1 = fma((double)t.y, rb, eb * (double)vev.y);
                const double t2 = fma((double)t.z, rb, eb * (double)vev.z);
                const double t3 = fma((double)t.w, rb, eb * (double)vev.w);
                th[idx] = make_float4((float)t0, (float)t1, (float)t2, (float)t3);
                acc[h][0] = fma(gb, t0, acc[h][0]);
                acc[h][1] = fma(gb, t1, acc[h][1]);
                acc[h][2] = fma(gb, t2, acc[h][2]);
                acc[h][3] = fma(gb, t3, acc[h][3]);
            }
        }
    }
    {
#pragma unroll 4
        for (int r = rl; r < R; r += C::RL) {
            const float4 x = (r == slot_row) ? vn_s[cc] : nv[(size_t)r * C::VCH + cc];
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                const double p = lg_s[h * R + r];
                acc[h][0] = fma(p, (double)x.x, acc[h][0]);
                acc[h][1] = fma(p, (double)x.y, acc[h][1]);
                acc[h][2] = fma(p, (double)x.z, acc[h][2]);
                acc[h][3] = fma(p, (double)x.w, acc[h][3]);
            }
        }
    }

    // ---- 5. reduce row lanes, joint division, counters --------------------
    float4 *outp = reinterpret_cast<float4 *>(io.out) + gh0 * C::VCH;
#pragma unroll
    for (int h = 0; h < HPK; ++h) {
        red_s[rl][cc * 4 + 0] = acc[h][0];
        red_s[rl][cc * 4 + 1] = acc[h][1];
        red_s[rl][cc * 4 + 2] = acc[h][2];
        red_s[rl][cc * 4 + 3] = acc[h][3];
        __syncthreads();
        if (tid < C::VCH) {
            double o0 = 0.0, o1 = 0.0, o2 = 0.0, o3 = 0.0;
#pragma unroll
            for (int j = 0; j < C::RL; ++j) {
                o0 += red_s[j][tid * 4 + 0];
                o1 += red_s[j][tid * 4 + 1];
                o2 += red_s[j][tid * 4 + 2];
                o3 += red_s[j][tid * 4 + 3];
            }
            const double den = fmax(den_s[h], kDenEps);
            outp[(size_t)h * C::VCH + tid] =
                make_float4((float)(o0 / den), (float)(o1 / den), (float)(o2 / den), (float)(o3 / den));
        }
        __syncthreads();
    }
    if (tid == 0) s.win_head[g] = (e + 1 == s.w) ? 0 : e + 1;
    if (tid < HPK) s.far_len[gh0 + tid] += 1;
}

template <int D, int DV, int HPK>
hipError_t launch_shape(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    const size_t dyn = sizeof(double) * (size_t)HPK * s.R;
    hipLaunchKernelGGL((decode_kernel<D, DV, HPK>), dim3(s.G), dim3(kThreads), dyn, stream, s, io);
    return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_hpk(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    switch (s.hpk) {
    case 1: return launch_shape<D, DV, 1>(s, io, stream);
    case 2: return launch_shape<D, DV, 2>(s, io, stream);
    case 4: return launch_shape<D, DV, 4>(s, io, stream);
    case 8: return launch_shape<D, DV, 8>(s, io, stream);
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
    return (size_t)hpk * R * sizeof(double) <= 32 * 1024;
}

hipError_t launch_decode(const DevState &s, const DecodeIO &io, hipStream_t stream)
{
    if (!decode_supported(s.d, s.dv, s.hpk, s.m, s.R)) return hipErrorInvalidValue;
    if (s.d == 64) return launch_hpk<64, 64>(s, io, stream);
    return launch_hpk<128, 128>(s, io, stream);
}

}  // namespace o1
