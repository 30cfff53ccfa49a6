// Exact grouped-GQA decode attention over a stored KV cache: the comparator the
// O(1) operator replaces (LayerKvCache::attend_group on the docs.rs LayerKvCache
// page: all query heads of one KV group in one pass over the stored K rows and
// one pass over the V rows; keys before `first` get zero probability).
//
//   out_h = sum_{j in [first, n_keys)} softmax_j(q_h . k_j * scale) v_j
//
// exact_attend_kernel: grid (G, splits), 512 threads for one or two query heads,
// 256 for more.  A work-group owns one
// key range of one group and walks it in chunks of kChunk keys with an online
// per-head max: row-dot pass (f64, the decode kernel's lane split and head
// reduction; the chunk's first V rows of each lane are loaded at its end, so
// they arrive during the softmax) -> per-head chunk max, weights and running
// sum -> V pass with the running rescale.  With one split it writes the normalised output; otherwise
// it writes (max, sum, numerator) partials that exact_combine_kernel merges.
// Bound: HBM (n_keys * (d + dv) * 4 B per group, read once, nontemporal).
//
// In append mode (the exact-only decode step of NystromState::step_group: the
// new key joins the window before any output) the last key comes from k_new /
// v_new; the work-group whose range holds it also stores it into the cache, and
// no other work-group reads that row.
#include "o1_internal.h"

namespace o1 {
namespace {

constexpr int kChunk = 256;     // keys a work-group walks per step of its online softmax
constexpr int kSplitKeys = 128; // fewest keys per work-group when a range is split

template <int D, int DV, int HPK>
struct ExactShape {
    // one or two query heads: 512 threads (twice the rows per round trip on
    // short key ranges) held to 128 VGPRs so that two work-groups share a CU's
    // SIMDs; more heads need the registers of a 256-thread work-group
    static constexpr int NT = HPK <= 2 ? 512 : 256;
    static constexpr int NW = NT / 64;
    static constexpr int CH = D / 4;
    static constexpr int LPR_WANT = HPK <= 2 ? 8 : (HPK <= 4 ? 16 : 32);
    static constexpr int LPR = pow2_divisor(LPR_WANT, CH);
    static constexpr int CPL = CH / LPR;
    static constexpr int RPW = 64 / LPR;
    static constexpr int RPB = RPW * NW;
    static constexpr int UNR = CPL >= 8 ? 1 : (CPL >= 4 ? 2 : (CPL == 3 ? 3 : (CPL == 2 ? 4 : 8)));
    // (more than 9 key float4 in flight per lane, as 192-float keys take,
    // do not fit the registers of four waves per SIMD)
    static constexpr int WAVES_PER_SIMD =
        HPK <= 2 ? (UNR * CPL > 9 ? 2 : 4) : (HPK == 8 && D % 16 == 0 && D <= 128 ? 2 : 1);
    static constexpr int VCH = DV / 4;
    static constexpr int VCP = pow2_ceil(VCH);  // lanes per value row (VCH used)
    static constexpr int RL = NT / VCP;
    static constexpr int RED_CAP = pow2_floor(16384 / (NW * DV * 8));
    static constexpr int RED_H = HPK < RED_CAP ? HPK : RED_CAP;
    // V rows per lane loaded before the chunk's softmax (more would cost a wave
    // per SIMD at hpk >= 4)
    static constexpr int VPRE = HPK <= 2 && DV <= 128 ? 8 : 4;
    // eight heads: the key dots on f64 MFMA (16-key tiles times the queries)
    // instead of per-lane dots and 32-lane head reductions
    static constexpr bool MFMA_ROWS = HPK == 8 && D % 16 == 0 && D <= 128;
    static_assert(HPK <= LPR && HPK % RED_H == 0, "unsupported head count");
};

template <int D, int DV, int HPK>
__global__ __launch_bounds__((ExactShape<D, DV, HPK>::NT))
__attribute__((amdgpu_waves_per_eu(ExactShape<D, DV, HPK>::WAVES_PER_SIMD))) void exact_attend_kernel(ExactIO a)
{
    using C = ExactShape<D, DV, HPK>;
    constexpr int kNT = C::NT, kNW = C::NW;
    const int ci = blockIdx.x, sp = blockIdx.y;  // call index (q, out, new key, partials)
    const int g = a.map.state(ci);              // cache group
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int n_keys = a.n_keys, per_split = a.per_split;
    if (a.held) {  // exact-only decode: this group's key count from the device
        const int held = a.held[g];
        if (held >= a.cap) return;  // full: the step changes nothing here
        n_keys = held + 1;
        per_split = (n_keys - a.first + (int)gridDim.y - 1) / (int)gridDim.y;
    }
    const int k0 = a.first + sp * per_split;
    const int k1 = min(k0 + per_split, n_keys);
    const double scale = (double)a.scale;
    const double NEG_INF = -__builtin_inf();

    __shared__ float4 q_s[HPK][C::CH];
    __shared__ double lg_s[HPK][kChunk];
    __shared__ double fac_s[HPK];
    __shared__ double red_s[kNW][C::RED_H * DV];

    // query heads: HPK is the compiled count (a power of two), H the group's own
    // (HPK / 2 < H <= HPK); heads H .. HPK-1 take zero queries and write nothing
    const int H = a.hpk;
    const size_t gh0 = (size_t)ci * a.hg + a.h0;  // first head of this block
    const float4 *qg = reinterpret_cast<const float4 *>(a.q) + gh0 * C::CH;
    for (int i = tid; i < HPK * C::CH; i += kNT)
        (&q_s[0][0])[i] = i < H * C::CH ? qg[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 *kc = reinterpret_cast<const float4 *>(a.k) + (size_t)g * a.cap * C::CH;
    const float4 *vc = reinterpret_cast<const float4 *>(a.v) + (size_t)g * a.cap * C::VCH;
    const int new_row = a.k_new ? n_keys - 1 : -1;  // absolute index of the appended key
    const float4 *kn = reinterpret_cast<const float4 *>(a.k_new) + (size_t)ci * C::CH;
    const float4 *vn = reinterpret_cast<const float4 *>(a.v_new) + (size_t)ci * C::VCH;
    if (a.shared && new_row >= k0 && new_row < k1) {
        if (tid < C::CH) reinterpret_cast<float4 *>(a.k_dst)[((size_t)g * a.cap + new_row) * C::CH + tid] = kn[tid];
        if (tid >= 128 && tid < 128 + C::VCH)
            reinterpret_cast<float4 *>(a.v_dst)[((size_t)g * a.cap + new_row) * C::VCH + tid - 128] = vn[tid - 128];
    }

    const int sub = lane % C::LPR, rsub = lane / C::LPR;
    constexpr int HSTRIDE = C::LPR / HPK;
    const int my_head = sub / HSTRIDE;
    const bool writer = (sub % HSTRIDE) == 0;
    // V pass: column lane cp of row lane rl; lanes past a row's VCH columns (VCH
    // not a power of two) repeat its last column and store nothing
    const int cp = tid % C::VCP, rl = tid / C::VCP, cc = min(cp, C::VCH - 1);

    constexpr int HPW = (HPK + kNW - 1) / kNW;  // heads per wave: h = wave + j * kNW
    double run_max[HPW], run_sum[HPW];          // running max / sum of the wave's heads
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
        run_max[j] = NEG_INF;
        run_sum[j] = 0.0;
    }
    double acc[HPK][4];
#pragma unroll
    for (int h = 0; h < HPK; ++h) acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.0;
    __syncthreads();

    for (int c0 = k0; c0 < k1; c0 += kChunk) {
        const int nr = min(kChunk, k1 - c0);
        // row dots of this chunk's keys
        if constexpr (C::MFMA_ROWS) {
            // eight heads: 16-key tiles times B = [q_0 .. q_7, 0 ..] on f64
            // MFMA.  Operand layout (wave64): A[i][k] in lane i + 16 k, B[k][j]
            // in lane j + 16 k; f64 D[i][j] in lane j + 16 (i % 4), element
            // i / 4.  In step (jj, c) k-lane kk stands for component
            // 16 jj + 4 kk + c of A and B alike, so a lane's operands of one
            // key are the D/16 float4 at 4 jj + kk.  Keys past the chunk load
            // its last key and are discarded.
            constexpr int NJ = D / 16;
            using d4v = __attribute__((ext_vector_type(4))) double;
            const int li = lane & 15, lk = lane >> 4;
            // column li of B: head li's query (read from LDS at each step, so
            // it holds no registers), zero past the heads
            const float4 *bq = &q_s[min(li, HPK - 1)][lk];
            const float bm = li < HPK ? 1.0f : 0.0f;
            const int ntile = (nr + 15) / 16;
            auto load = [&](float4 (&x)[NJ], int t) {
                const int r = c0 + min(16 * t + li, nr - 1);
                const float4 *row = (r == new_row) ? kn : kc + (size_t)r * C::CH;
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) x[jj] = ld4<true>(row + 4 * jj + lk);
            };
            auto mma = [&](float4 (&x)[NJ], int t) {
                d4v acc = {0.0, 0.0, 0.0, 0.0}, acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int jj = 0; jj < NJ; ++jj) {
                    const float4 b = bq[4 * jj];
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].x, (double)(b.x * bm), acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].y, (double)(b.y * bm), acc2, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].z, (double)(b.z * bm), acc, 0, 0, 0);
                    acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64((double)x[jj].w, (double)(b.w * bm), acc2, 0, 0, 0);
                }
                acc += acc2;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * t + 4 * e + lk;  // D[4 e + lk][li]
                    if (li < HPK && r < nr) lg_s[li][r] = acc[e] * scale;
                }
            };
            for (int t = wave; t < ntile; t += kNW) {
                float4 xa[NJ];
                load(xa, t);
                mma(xa, t);
            }
        } else
        for (int base = wave * C::RPW; base < nr; base += C::UNR * C::RPB) {
            float4 x[C::UNR][C::CPL];
#pragma unroll
            for (int u = 0; u < C::UNR; ++u) {
                const int r = c0 + min(base + u * C::RPB + rsub, nr - 1);
                const float4 *row = (r == new_row) ? kn : kc + (size_t)r * C::CH;
#pragma unroll
                for (int k = 0; k < C::CPL; ++k) x[u][k] = ld4<true>(row + sub + C::LPR * k);
            }
#pragma unroll
            for (int u = 0; u < C::UNR; ++u) {
                const int r = base + u * C::RPB + rsub;
                double part[HPK];
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    asm volatile("" ::: "memory");
                    double s = 0.0;
#pragma unroll
                    for (int k = 0; k < C::CPL; ++k) s += dot4(q_s[h][sub + C::LPR * k], x[u][k]);
                    part[h] = s;
                }
                const double tot = head_reduce<C::LPR, HPK>(part, lane) * scale;
                if (writer && r < nr) lg_s[my_head][r] = tot;
            }
        }
        // the chunk's first V rows of this lane, in flight across the softmax
        float4 vp[C::VPRE];
#pragma unroll
        for (int j = 0; j < C::VPRE; ++j) {
            const int r = c0 + min(rl + j * C::RL, nr - 1);
            vp[j] = ld4<true>(((r == new_row) ? vn : vc + (size_t)r * C::VCH) + cc);
        }
        __syncthreads();
        // per head: chunk max, running rescale, weights
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
            const int h = wave + j * kNW;
            if (h >= HPK) break;
            double cm = NEG_INF;
            for (int r = lane; r < nr; r += 64) cm = fmax(cm, lg_s[h][r]);
            cm = wave_max(cm);
            const double nm = fmax(run_max[j], cm);
            const double f = exp(run_max[j] - nm);  // 0 on the first chunk
            double ps = 0.0;
            for (int r = lane; r < nr; r += 64) {
                const double p = exp(lg_s[h][r] - nm);
                lg_s[h][r] = p;
                ps += p;
            }
            ps = wave_sum(ps);
            run_sum[j] = run_sum[j] * f + ps;
            run_max[j] = nm;
            if (lane == 0) fac_s[h] = f;
        }
        __syncthreads();
        // V pass with the running rescale
#pragma unroll
        for (int h = 0; h < HPK; ++h) {
            const double f = fac_s[h];
            acc[h][0] *= f;
            acc[h][1] *= f;
            acc[h][2] *= f;
            acc[h][3] *= f;
        }
#pragma unroll
        for (int j = 0; j < C::VPRE; ++j) {
            const int r = rl + j * C::RL;
            if (r >= nr) break;
#pragma unroll
            for (int h = 0; h < HPK; ++h) {
                const double p = lg_s[h][r];
                acc[h][0] = fma(p, (double)vp[j].x, acc[h][0]);
                acc[h][1] = fma(p, (double)vp[j].y, acc[h][1]);
                acc[h][2] = fma(p, (double)vp[j].z, acc[h][2]);
                acc[h][3] = fma(p, (double)vp[j].w, acc[h][3]);
            }
        }
        constexpr int VU = 8;
        for (int r0 = rl + C::VPRE * C::RL; r0 < nr; r0 += VU * C::RL) {
            float4 x[VU];
#pragma unroll
            for (int j = 0; j < VU; ++j) {
                const int r = c0 + min(r0 + j * C::RL, nr - 1);
                x[j] = ld4<true>(((r == new_row) ? vn : vc + (size_t)r * C::VCH) + cc);
            }
            // many heads or wide rows: the rows are taken as loaded here, as
            // the compiler otherwise sinks each load past the exit test below
            // to its use and waits for it alone (with fewer heads it keeps
            // them in flight and adds each in as it arrives)
            if constexpr (HPK >= 4 || DV > 128) {
#pragma unroll
                for (int j = 0; j < VU; ++j) asm volatile("" : "+v"(x[j].x), "+v"(x[j].y), "+v"(x[j].z), "+v"(x[j].w));
            }
#pragma unroll
            for (int j = 0; j < VU; ++j) {
                const int r = r0 + j * C::RL;
                if (r >= nr) break;
#pragma unroll
                for (int h = 0; h < HPK; ++h) {
                    const double p = lg_s[h][r];
                    acc[h][0] = fma(p, (double)x[j].x, acc[h][0]);
                    acc[h][1] = fma(p, (double)x[j].y, acc[h][1]);
                    acc[h][2] = fma(p, (double)x[j].z, acc[h][2]);
                    acc[h][3] = fma(p, (double)x[j].w, acc[h][3]);
                }
            }
        }
        __syncthreads();
    }

    // running max / sum of each head into LDS for every thread
    __shared__ double hmax_s[HPK], hsum_s[HPK];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
        const int h = wave + j * kNW;
        if (h < HPK && lane == 0) {
            hmax_s[h] = run_max[j];
            hsum_s[h] = run_sum[j];
        }
    }
    // reduce the row lanes: shuffles inside a wave, then LDS across waves
#pragma unroll
    for (int h = 0; h < HPK; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[h][c] = sum_high_lanes<C::VCP>(acc[h][c]);
    const bool final_out = gridDim.y == 1;
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
        if (tid < C::RED_H * C::VCH && h0 + tid / C::VCH < H) {
            const int hh = tid / C::VCH, c4 = tid - hh * C::VCH, h = h0 + hh;
            double o[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int j = 0; j < kNW; ++j)
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] += red_s[j][hh * DV + c4 * 4 + c];
            if (final_out) {
                const double den = hsum_s[h];
                reinterpret_cast<float4 *>(a.out)[(gh0 + h) * C::VCH + c4] =
                    make_float4((float)(o[0] / den), (float)(o[1] / den), (float)(o[2] / den),
                                (float)(o[3] / den));
            } else {
                const size_t part = ((size_t)ci * gridDim.y + sp) * H + h;
                double *num = a.ws_num + part * DV + c4 * 4;
                num[0] = o[0];
                num[1] = o[1];
                num[2] = o[2];
                num[3] = o[3];
                if (c4 == 0) {
                    a.ws_max[part] = hmax_s[h];
                    a.ws_sum[part] = hsum_s[h];
                }
            }
        }
        if (h0 + C::RED_H < HPK) __syncthreads();
    }
    // exact-only decode with one work-group per group: it alone read the count
    // (at its start), so it advances it; split ranges leave that to the merge
    if (a.held && a.shared && final_out && tid == 0) a.held[g] = n_keys;
}

// One block of dv threads per call index: merge the key-range partials of
// every head.  In the exact-only decode the block also advances the group's
// key count, after every thread has read it.
__global__ void exact_combine_kernel(ExactIO a, int splits)
{
    const int ci = blockIdx.x, H = a.hpk, c = threadIdx.x;
    const int g = a.map.state(ci);
    int held = 0;
    if (a.held) {
        held = a.held[g];
        if (held >= a.cap) return;  // as the attention: full, nothing changes
    }
    for (int h = 0; h < H; ++h) {
        double mx = -__builtin_inf();
        for (int s = 0; s < splits; ++s) mx = fmax(mx, a.ws_max[((size_t)ci * splits + s) * H + h]);
        double den = 0.0, num = 0.0;
        for (int s = 0; s < splits; ++s) {
            const size_t part = ((size_t)ci * splits + s) * H + h;
            const double w = exp(a.ws_max[part] - mx);  // empty ranges carry -inf -> 0
            den += a.ws_sum[part] * w;
            num += a.ws_num[part * a.dv + c] * w;
        }
        a.out[((size_t)ci * a.hg + a.h0 + h) * a.dv + c] = (float)(num / den);
    }
    if (a.held && a.shared) {
        __syncthreads();  // every thread has read the count
        if (c == 0) a.held[g] = held + 1;
    }
}

template <int D, int DV, int HPK>
hipError_t launch_exact_shape(const ExactIO &a, int splits, hipStream_t stream)
{
    hipLaunchKernelGGL((exact_attend_kernel<D, DV, HPK>), dim3(a.map.count, splits),
                       dim3(ExactShape<D, DV, HPK>::NT), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || splits == 1) return err;
    hipLaunchKernelGGL(exact_combine_kernel, dim3(a.map.count), dim3(a.dv), 0, stream, a, splits);
    return hipGetLastError();
}

template <int D, int DV>
hipError_t launch_exact_hpk(const ExactIO &a, int splits, hipStream_t stream)
{
    // hpk heads run the kernel compiled for the next power of two
    switch (a.hpk) {
    case 1: return launch_exact_shape<D, DV, 1>(a, splits, stream);
    case 2: return launch_exact_shape<D, DV, 2>(a, splits, stream);
    case 3:
    case 4: return launch_exact_shape<D, DV, 4>(a, splits, stream);
    case 5:
    case 6:
    case 7:
    case 8:
        if constexpr (block_heads(D) >= 8) return launch_exact_shape<D, DV, 8>(a, splits, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

// One work-group per call index: copy the prompt rows into the mapped group's
// exact buffers and clear the counters the skeleton mode would have set.
__global__ __launch_bounds__(256) void exact_seal_kernel(DevState s, PromptView p, GroupMap map, int T,
                                                         float4 *ek, float4 *ev, int cap, int32_t *held)
{
    const int ci = blockIdx.x, g = map.state(ci), tid = threadIdx.x;
    if (tid == 0) held[g] = T;
    const int ck = s.d / 4, cv = s.dv / 4;
    const float4 *k = reinterpret_cast<const float4 *>(p.k_row(map, ci, 0));
    const float4 *v = reinterpret_cast<const float4 *>(p.v_row(map, ci, 0));
    const int64_t kp = p.k_pos / 4, vp = p.v_pos / 4;
    for (int i = tid; i < T * ck; i += 256) {
        const int t = i / ck, c = i - t * ck;
        ek[((size_t)g * cap + t) * ck + c] = k[(int64_t)t * kp + c];
    }
    for (int i = tid; i < T * cv; i += 256) {
        const int t = i / cv, c = i - t * cv;
        ev[((size_t)g * cap + t) * cv + c] = v[(int64_t)t * vp + c];
    }
    if (tid == 0) s.win_head[g] = 0;
    if (tid < s.hpk) {
        const size_t gh = (size_t)g * s.hpk + tid;
        s.far_len[gh] = 0;
        s.lambda[gh] = 0.0;
        s.tries[gh] = 0;
    }
}

}  // namespace

hipError_t launch_exact_seal(const DevState &s, const PromptView &p, const GroupMap &map, int T,
                             float *ek, float *ev, int cap, int32_t *held, hipStream_t stream)
{
    hipLaunchKernelGGL(exact_seal_kernel, dim3(map.count), dim3(256), 0, stream, s, p, map, T,
                       reinterpret_cast<float4 *>(ek), reinterpret_cast<float4 *>(ev), cap, held);
    return hipGetLastError();
}

int exact_splits(int G, int n_visible)
{
    // enough work-groups to cover the CUs several times, at least kSplitKeys keys each
    const int want = (4 * 256 + G - 1) / G;
    const int most = (n_visible + kSplitKeys - 1) / kSplitKeys;
    int s = want < most ? want : most;
    return s < 1 ? 1 : s;
}

hipError_t launch_exact(const ExactIO &in, int splits, hipStream_t stream)
{
    // groups of more heads than a block holds (block_heads): one launch (and merge) per
    // block of heads, in order; the last stores the appended key and advances
    // the count, so every earlier block still reads the count it started from
    const int bh = block_heads(in.d);
    for (int h0 = 0; h0 < in.hpk; h0 += bh) {
        ExactIO a = in;
        a.hg = in.hpk;
        a.h0 = h0;
        a.hpk = min(bh, in.hpk - h0);
        a.shared = h0 + bh >= in.hpk;
        hipError_t err;
        if (a.d == 64 && a.dv == 64) err = launch_exact_hpk<64, 64>(a, splits, stream);
        else if (a.d == 96 && a.dv == 96) err = launch_exact_hpk<96, 96>(a, splits, stream);
        else if (a.d == 128 && a.dv == 128) err = launch_exact_hpk<128, 128>(a, splits, stream);
        else if (a.d == 256 && a.dv == 256) err = launch_exact_hpk<256, 256>(a, splits, stream);
        else if (a.d == 192 && a.dv == 128) err = launch_exact_hpk<192, 128>(a, splits, stream);
        else if (a.d == 80 && a.dv == 80) err = launch_exact_hpk<80, 80>(a, splits, stream);
        else err = hipErrorInvalidValue;
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace o1
