// Bounds kernels: key mean, centred key radii, norms and per-head eligibility.
//
// Source: "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
// (news.xcc.im/article/5328), "Unchaining the Softmax" ¶2-¶3. By
// Cauchy-Schwarz a row's largest logit is at most its query norm times the
// largest key norm; centring the keys on their mean first leaves the softmax
// unchanged and tightens that bound; with windowed slices the key maximum is
// taken over the row's own slice; heads whose bound is too loose are flagged
// for the online route.
//
// HBM-bound: K is read twice (mean, then the radii of the centred keys) and Q
// once; nothing of the size of K is written. The key side is the chunk's own
// frames (self-attention) or a separate set of M reference tokens that every
// query attends to (cross-attention: one key frame, one radius per head). The
// centred keys themselves are never stored: the forward pass scores K as given
// and moves each row's shift by scale * q.mu instead. Every reduction is deterministic: sums in a fixed
// order, maxima exact.
#include <hip/hip_runtime.h>

#include "fsa_internal.h"

namespace {

using fsa::FrameTable;

template <typename E>
struct Pack16 {                      // one 16-byte vector of E
    static constexpr int n = 16 / sizeof(E);
    E v[n];
};

template <typename E>
__device__ __forceinline__ Pack16<E> load16(const E* p) {
    Pack16<E> r;
    *reinterpret_cast<uint4*>(r.v) = *reinterpret_cast<const uint4*>(p);
    return r;
}

template <typename E>
__device__ __forceinline__ void store16(E* p, const Pack16<E>& r) {
    *reinterpret_cast<uint4*>(p) = *reinterpret_cast<const uint4*>(r.v);
}

// Parts as the kernels read them (fsa::Parts without its host helpers).
struct PartsArg {
    int span, rows_per_part, per_frame, count;
};

PartsArg parts_arg(const fsa::Parts& g) { return {g.span, g.rows_per_part, g.per_frame, g.count()}; }

// Rows of one workgroup: part `part` of one side, never crossing a frame.
struct PartRows {
    int begin, end;
};

__device__ __forceinline__ PartRows part_rows(int part, const PartsArg& g) {
    const int frame = part / g.per_frame, sub = part % g.per_frame;
    PartRows r;
    r.begin = frame * g.span + sub * g.rows_per_part;
    r.end = min(frame * g.span + g.span, r.begin + g.rows_per_part);
    return r;
}

// Pass 1: per-part column sums of K (for the mean) and row norms of Q.
// JOINT: the query and key sides share one part geometry (self-attention),
// and each workgroup reads its rows of Q and K in the same loop. Otherwise
// workgroup `part` reduces key part `part` and query part `part`, each where
// it exists.
template <typename E, int D, bool JOINT>
__global__ __launch_bounds__(256) void bounds_colsum_qnorm(
    const E* __restrict__ Q, const E* __restrict__ K, float* __restrict__ colsum,
    float* __restrict__ qnorm, float* __restrict__ partqmax, int N, int NK, PartsArg qp,
    PartsArg kp) {
    constexpr int V = Pack16<E>::n;
    constexpr int LPR = D / V;        // lanes per row
    constexpr int RPI = 256 / LPR;    // rows per iteration
    __shared__ float red[RPI][D];
    __shared__ float qred[RPI];

    const int part = blockIdx.x, bh = blockIdx.y;
    const int lane = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
    const E* Qh = Q + size_t(bh) * N * D;
    const E* Kh = K + size_t(bh) * NK * D;
    const bool has_k = part < kp.count, has_q = part < qp.count;   // uniform

    float acc[V];
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = 0.f;
    float qbest = 0.f;
    auto qrow = [&](int r) {
        const Pack16<E> q = load16(Qh + size_t(r) * D + lane * V);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float qe = float(q.v[e]);
            ss = fmaf(qe, qe, ss);
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        const float qn = sqrtf(ss);
        qbest = fmaxf(qbest, qn);
        if (lane == 0) qnorm[size_t(bh) * N + r] = qn;
    };
    auto krow = [&](int r) {
        const Pack16<E> k = load16(Kh + size_t(r) * D + lane * V);
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += float(k.v[e]);
    };
    if (JOINT) {
        const PartRows pr = part_rows(part, qp);
        int r = pr.begin + r0;
        // four rows a trip, their loads issued together
        for (; r + 3 * RPI < pr.end; r += 4 * RPI) {
            Pack16<E> kk[4], qq[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kk[u] = load16(Kh + size_t(r + u * RPI) * D + lane * V);
                qq[u] = load16(Qh + size_t(r + u * RPI) * D + lane * V);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int e = 0; e < V; ++e) acc[e] += float(kk[u].v[e]);
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < V; ++e) {
                    const float qe = float(qq[u].v[e]);
                    ss = fmaf(qe, qe, ss);
                }
#pragma unroll
                for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
                const float qn = sqrtf(ss);
                qbest = fmaxf(qbest, qn);
                if (lane == 0) qnorm[size_t(bh) * N + r + u * RPI] = qn;
            }
        }
        for (; r < pr.end; r += RPI) {
            krow(r);
            qrow(r);
        }
    } else {
        if (has_k) {
            const PartRows pr = part_rows(part, kp);
            for (int r = pr.begin + r0; r < pr.end; r += RPI) krow(r);
        }
        if (has_q) {
            const PartRows pr = part_rows(part, qp);
            for (int r = pr.begin + r0; r < pr.end; r += RPI) qrow(r);
        }
    }
#pragma unroll
    for (int e = 0; e < V; ++e) red[r0][lane * V + e] = acc[e];
    if (lane == 0) qred[r0] = qbest;
    __syncthreads();
    if (threadIdx.x < D && has_k) {
        float s = 0.f;
        for (int i = 0; i < RPI; ++i) s += red[i][threadIdx.x];
        colsum[(size_t(bh) * kp.count + part) * D + threadIdx.x] = s;
    }
    if (threadIdx.x == D && has_q) {
        float b = 0.f;
        for (int i = 0; i < RPI; ++i) b = fmaxf(b, qred[i]);
        partqmax[size_t(bh) * qp.count + part] = b;
    }
}

// Pass 2: the key mean of each (batch, head), summing the parts in order.
template <int D>
__global__ __launch_bounds__(256) void bounds_mean(const float* __restrict__ colsum,
                                                   float* __restrict__ mu, int NK, int nparts) {
    const int bh = blockIdx.x, t = threadIdx.x;
    if (t >= D) return;
    float s = 0.f;
    const float* col = colsum + size_t(bh) * nparts * D + t;
#pragma unroll 16       // loads issue ahead; the additions keep their order
    for (int p = 0; p < nparts; ++p) s += col[size_t(p) * D];
    mu[size_t(bh) * D + t] = s / float(NK);
}

// Pass 3: the part's largest ||k_j - mu||, in fp32 from the keys as given.
template <typename E, int D>
__global__ __launch_bounds__(256) void bounds_radius(
    const E* __restrict__ K, const float* __restrict__ mu, float* __restrict__ partmax, int NK,
    PartsArg kp) {
    constexpr int V = Pack16<E>::n;
    constexpr int LPR = D / V;
    constexpr int RPI = 256 / LPR;
    __shared__ float red[RPI];

    const int part = blockIdx.x, bh = blockIdx.y;
    const PartRows pr = part_rows(part, kp);
    const int lane = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
    const E* Kh = K + size_t(bh) * NK * D;

    float m[V];
#pragma unroll
    for (int e = 0; e < V; ++e) m[e] = mu[size_t(bh) * D + lane * V + e];
    float best = 0.f;
    int r = pr.begin + r0;
    for (; r + 3 * RPI < pr.end; r += 4 * RPI) {       // four rows a trip, loads together
        Pack16<E> kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kk[u] = load16(Kh + size_t(r + u * RPI) * D + lane * V);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < V; ++e) {
                const float ce = float(kk[u].v[e]) - m[e];
                ss = fmaf(ce, ce, ss);
            }
#pragma unroll
            for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
            best = fmaxf(best, sqrtf(ss));
        }
    }
    for (; r < pr.end; r += RPI) {
        const Pack16<E> k = load16(Kh + size_t(r) * D + lane * V);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float ce = float(k.v[e]) - m[e];
            ss = fmaf(ce, ce, ss);
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
        best = fmaxf(best, sqrtf(ss));
    }
    if (lane == 0) red[r0] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = 0.f;
        for (int i = 0; i < RPI; ++i) b = fmaxf(b, red[i]);
        partmax[size_t(bh) * kp.count + part] = b;
    }
}

// Pass 4, per (batch, head): per-key-frame radius, per-slice radius, the
// largest row bound scale * ||q_i|| * R_S(f(i)) and the eligibility flag.
// Maxima are exact, so any reduction order gives the same bits. The largest
// row bound of frame f is (scale * max ||q_i||) * R_S(f): rounding is monotone.
__global__ __launch_bounds__(256) void bounds_finalize(
    const float* __restrict__ partqmax, const float* __restrict__ partmax,
    float* __restrict__ rframe, float* __restrict__ rslice, float* __restrict__ stat,
    uint8_t* __restrict__ elig, float* __restrict__ statf, uint8_t* __restrict__ eligf,
    unsigned* __restrict__ pmax, int F, int KF, PartsArg qp, PartsArg kp, float scale,
    const FrameTable tab) {
    __shared__ float rf[FSA_MAX_FRAMES + 1];
    __shared__ float qm[FSA_MAX_FRAMES + 1];
    __shared__ float sb[FSA_MAX_FRAMES + 1];
    const int bh = blockIdx.x;
    if (bh == 0 && threadIdx.x == 0) *pmax = 0u;      // forward's probability record starts over
    for (int g = threadIdx.x; g < KF; g += blockDim.x) {
        float b = 0.f;
        for (int s = 0; s < kp.per_frame; ++s)
            b = fmaxf(b, partmax[size_t(bh) * kp.count + g * kp.per_frame + s]);
        rf[g] = b;
        rframe[size_t(bh) * KF + g] = b;
    }
    for (int f = threadIdx.x; f < F; f += blockDim.x) {
        float q = 0.f;
        for (int s = 0; s < qp.per_frame; ++s)
            q = fmaxf(q, partqmax[size_t(bh) * qp.count + f * qp.per_frame + s]);
        qm[f] = q;
    }
    __syncthreads();
    for (int f = threadIdx.x; f < F; f += blockDim.x) {
        const uint32_t run = tab.runs[f];
        const int a0 = run & 0xff, l0 = (run >> 8) & 0xff;
        const int a1 = (run >> 16) & 0xff, l1 = run >> 24;
        float r = 0.f;
        for (int g = a0; g < a0 + l0; ++g) r = fmaxf(r, rf[g]);
        for (int g = a1; g < a1 + l1; ++g) r = fmaxf(r, rf[g]);
        rslice[size_t(bh) * F + f] = r;
        sb[f] = (scale * qm[f]) * r;
        statf[size_t(bh) * F + f] = sb[f];
        eligf[size_t(bh) * F + f] = sb[f] <= FSA_ELIG_BETA ? 1 : 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float st = 0.f;
        for (int f = 0; f < F; ++f) st = fmaxf(st, sb[f]);
        stat[bh] = st;
        elig[bh] = st <= FSA_ELIG_BETA ? 1 : 0;
    }
}

// Pass 5, per (batch, head, query frame): the slice's mean key minus mu, from
// the per-part column sums (parts never straddle a key frame, so the parts of
// a run of key frames are one contiguous range). The gap bound of a row,
// B_i - scale q_i.(kbar_S - mu), is at least how far the fixed max lies above
// the row's largest logit, because a maximum is at least a mean. Parts are
// added in order (run 0, then run 1): a fixed summation order; loads issue
// eight ahead of the additions.
__device__ __forceinline__ float add_parts(const float* cs, int D, int p0, int p1, float s) {
    int p = p0;
    for (; p + 8 <= p1; p += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = cs[size_t(p + k) * D];
#pragma unroll
        for (int k = 0; k < 8; ++k) s += v[k];
    }
    for (; p < p1; ++p) s += cs[size_t(p) * D];
    return s;
}

__global__ __launch_bounds__(128) void bounds_slice_mean(
    const float* __restrict__ colsum, const float* __restrict__ mu, float* __restrict__ dslice,
    int F, int D, int KT, PartsArg kp, const FrameTable tab) {
    const int f = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
    if (t >= D) return;
    const uint32_t run = tab.runs[f];
    const int a0 = run & 0xff, l0 = (run >> 8) & 0xff;
    const int a1 = (run >> 16) & 0xff, l1 = run >> 24;
    const float* cs = colsum + size_t(bh) * kp.count * D + t;
    float s = add_parts(cs, D, a0 * kp.per_frame, (a0 + l0) * kp.per_frame, 0.f);
    s = add_parts(cs, D, a1 * kp.per_frame, (a1 + l1) * kp.per_frame, s);
    dslice[(size_t(bh) * F + f) * D + t] = s / float((l0 + l1) * KT) - mu[size_t(bh) * D + t];
}

template <typename E, int D>
fsa_status run_bounds(const fsa_plan& p, const void* Qv, const void* Kv, void* wsv, float scale,
                      hipStream_t stream) {
    const fsa_shape& s = p.shape;
    const int N = s.F * s.T, NK = int(p.key_tokens()), BH = s.B * s.H;
    const PartsArg qp = parts_arg(p.bounds.q), kp = parts_arg(p.bounds.k);
    char* ws = static_cast<char*>(wsv);
    const E* Q = static_cast<const E*>(Qv);
    const E* K = static_cast<const E*>(Kv);
    float* mu = reinterpret_cast<float*>(ws + p.ws.mu);
    float* qn = reinterpret_cast<float*>(ws + p.ws.qnorm);
    float* colsum = reinterpret_cast<float*>(ws + p.bounds.colsum);
    float* partmax = reinterpret_cast<float*>(ws + p.bounds.partmax);
    float* partqmax = reinterpret_cast<float*>(ws + p.bounds.partqmax);
    const bool joint = !p.cross;      // one part geometry for both sides
    const dim3 grid1(max(qp.count, kp.count), BH);
    if (joint)
        hipLaunchKernelGGL((bounds_colsum_qnorm<E, D, true>), grid1, dim3(256), 0, stream, Q, K,
                           colsum, qn, partqmax, N, NK, qp, kp);
    else
        hipLaunchKernelGGL((bounds_colsum_qnorm<E, D, false>), grid1, dim3(256), 0, stream, Q, K,
                           colsum, qn, partqmax, N, NK, qp, kp);
    hipLaunchKernelGGL((bounds_mean<D>), dim3(BH), dim3(256), 0, stream, colsum, mu, NK, kp.count);
    hipLaunchKernelGGL((bounds_radius<E, D>), dim3(kp.count, BH), dim3(256), 0, stream, K, mu,
                       partmax, NK, kp);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        fsa::set_error("fsa_bounds: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return fsa::launch_bounds_finalize(p, ws, scale, stream);
}

}  // namespace

namespace fsa {

fsa_status launch_bounds_finalize(const fsa_plan& p, char* ws, float scale, hipStream_t stream) {
    const fsa_shape& s = p.shape;
    const PartsArg qp = parts_arg(p.bounds.q), kp = parts_arg(p.bounds.k);
    hipLaunchKernelGGL(bounds_finalize, dim3(s.B * s.H), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(ws + p.bounds.partqmax),
                       reinterpret_cast<const float*>(ws + p.bounds.partmax),
                       reinterpret_cast<float*>(ws + p.ws.rframe),
                       reinterpret_cast<float*>(ws + p.ws.rslice),
                       reinterpret_cast<float*>(ws + p.ws.stat),
                       reinterpret_cast<uint8_t*>(ws + p.ws.elig),
                       reinterpret_cast<float*>(ws + p.ws.statf),
                       reinterpret_cast<uint8_t*>(ws + p.ws.eligf),
                       reinterpret_cast<unsigned*>(ws + p.ws.pmax), s.F, p.key_frames, qp, kp,
                       scale, p.table);
    hipLaunchKernelGGL(bounds_slice_mean, dim3(s.F, s.B * s.H), dim3(128), 0, stream,
                       reinterpret_cast<const float*>(ws + p.bounds.colsum),
                       reinterpret_cast<const float*>(ws + p.ws.mu),
                       reinterpret_cast<float*>(ws + p.ws.dslice), s.F, s.d, p.key_span, kp,
                       p.table);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("bounds: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return FSA_OK;
}

fsa_status launch_bounds(const fsa_plan& p, const void* Q, const void* K, void* ws, float scale,
                         hipStream_t stream) {
    const bool bf16 = p.shape.dtype == FSA_BF16;
    if (p.shape.d == 128)
        return bf16 ? run_bounds<__bf16, 128>(p, Q, K, ws, scale, stream)
                    : run_bounds<float, 128>(p, Q, K, ws, scale, stream);
    return bf16 ? run_bounds<__bf16, 64>(p, Q, K, ws, scale, stream)
                : run_bounds<float, 64>(p, Q, K, ws, scale, stream);
}

}  // namespace fsa
