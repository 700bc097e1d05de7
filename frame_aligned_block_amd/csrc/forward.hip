// Forward kernel: frame-aligned windowed attention, one launch.
//
// Source: "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
// (news.xcc.im/article/5328).
//  * "Deleting the Mask" ¶1-¶2: each frame's queries attend to a window of
//    frames plus a reference frame; blocks that are multiples of 16 tokens and
//    divide the frame span are entirely inside or outside the mask, so the
//    kernel visits only live keys, with no mask predicate and no padding, and
//    the reference frame is more full blocks in the same single pass.
//  * "Unchaining the Softmax" ¶2-¶3: each row's softmax shift is fixed in
//    advance at its Cauchy-Schwarz bound (no running max, no rescale chain);
//    heads whose bound is loose take the online softmax in the same kernel.
//  * "Proving the Pixels Didn't Change" ¶2: P enters the P.V product in bf16.
//
// gfx950 design (bf16):
//  * A workgroup is 4 waves; each wave owns 16*G consecutive query rows of one
//    frame, and the 4 waves of a workgroup own consecutive row units of the
//    same frame, so they share one key slice. The slice is at most two
//    contiguous token runs (the clipped window, and the reference frame when
//    it lies outside it), read from a per-frame table passed as a kernel
//    argument. The runs are walked as one sequence in chunks of 64 keys; only
//    the very last chunk can be shorter (16, 32 or 48 keys, a whole number of
//    16-key granules, so still no partial block).
//  * Per chunk, K (centred) and V are staged in LDS, double buffered with one
//    barrier per chunk; V is written transposed so the P.V operand is a
//    contiguous 16-byte read.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_bf16: the accumulator then holds, per lane, one query
//    and 4+4 keys, which is exactly the B-operand layout of O^T = V^T P^T, so P
//    never moves between lanes. Each lane also keeps one query's output
//    columns, so the row sum and the final division stay lane-local.
//  * Workgroups are numbered so that each XCD (8 per chip, one L2 each)
//    receives a contiguous range of (head, frame) work, heaviest frames first.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fsa_internal.h"

namespace {

using fsa::FrameTable;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;

struct FwdArgs {
    const void* Q;
    const void* Kc;             // centred keys (fixed-max route)
    const void* K;              // keys as given (online route)
    const void* V;
    void* O;
    const float* qnorm;
    const float* rslice;
    const uint8_t* elig;
    float c;                    // scale * log2(e)
    int32_t N, T, F, BH;
    int32_t units_per_frame;    // row units of 16*G rows per frame
    int32_t groups_per_frame;   // workgroups per (batch*head, frame)
    int32_t nwg;                // total workgroups
    int32_t mode;
    FrameTable tab;
};

// Hardware hands workgroup ids to the 8 XCDs round-robin. Renumber so XCD x
// runs a contiguous block of logical ids; a bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int hw, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = hw & 7, s = hw >> 3;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

__device__ __forceinline__ int frame_at(const FrameTable& t, int i) {
    return (t.order[i >> 2] >> (8 * (i & 3))) & 0xff;
}

struct Slice {
    int s0, n0, s1, total;      // tokens: run 0 = [s0, s0+n0), run 1 from s1
    __device__ __forceinline__ int key(int x) const { return x < n0 ? s0 + x : s1 + (x - n0); }
};

__device__ __forceinline__ Slice slice_of(const FrameTable& t, int f, int T) {
    const uint32_t run = t.runs[f];
    Slice s;
    s.s0 = int(run & 0xff) * T;
    s.n0 = int((run >> 8) & 0xff) * T;
    s.s1 = int((run >> 16) & 0xff) * T;
    s.total = s.n0 + int(run >> 24) * T;
    return s;
}

__device__ __forceinline__ bool use_fixed(const FwdArgs& p, int bh) {
    if (p.mode == FSA_MODE_FIXED_ONLY) return true;
    if (p.mode == FSA_MODE_ONLINE_ONLY) return false;
    return p.elig[bh] != 0;
}

// Position, within a 32-key group of the transposed V tile, of the 4-key
// group a (keys 4a..4a+3): lane group j of the P.V MFMA holds keys 4j..4j+3
// (slots 0-3) and 16+4j..16+4j+3 (slots 4-7) of the group.
__device__ __forceinline__ int vt_pos(int a) { return a < 4 ? 8 * a : 8 * (a - 4) + 4; }

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

// Workgroups per CU the register budget allows: two (<= 256 VGPRs per lane)
// while the per-wave state stays small, else one (up to 512 VGPRs + AGPRs).
constexpr int fwd_occupancy(int D, int G) { return D == 128 ? (G <= 2 ? 2 : 1) : (G <= 3 ? 2 : 1); }

template <int D, int G>
__global__ __launch_bounds__(fsa::kThreads, fwd_occupancy(D, G)) void fwd_bf16(const FwdArgs p) {
    constexpr int KS = D / 32;          // k-steps of S^T over d
    constexpr int DB = D / 16;          // 16-wide column blocks of O^T
    constexpr int BK = 64;              // keys per chunk
    constexpr int KROW = D * 2 + 16;    // bytes per K row in LDS (padded)
    constexpr int VROW = BK * 2 + 16;   // bytes per V^T row in LDS (padded)
    constexpr int KBYTES = BK * KROW;
    constexpr int STAGE = KBYTES + D * VROW;
    constexpr int KV16 = D / 8;         // 16-byte pieces per row
    constexpr int KPASS = BK * KV16 / fsa::kThreads;
    constexpr int KROWS_PER_PASS = fsa::kThreads / KV16;
    constexpr int VTASKS = (BK / 4) * KV16;   // (4 keys x 8 columns) tasks
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lj = lane >> 4;

    const int L = xcd_remap(blockIdx.x, p.nwg);
    const int gq = L % p.groups_per_frame;
    const int t1 = L / p.groups_per_frame;
    const int f = frame_at(p.tab, t1 % p.F);
    const int bh = t1 / p.F;
    const int T = p.T;
    const Slice sl = slice_of(p.tab, f, T);
    const int nchunks = (sl.total + BK - 1) / BK;

    const size_t base = size_t(bh) * p.N * D;
    const __bf16* Qh = static_cast<const __bf16*>(p.Q) + base;
    const bool fixed = use_fixed(p, bh);                 // uniform per workgroup
    const __bf16* Kh = static_cast<const __bf16*>(fixed ? p.Kc : p.K) + base;
    const __bf16* Vh = static_cast<const __bf16*>(p.V) + base;
    __bf16* Oh = static_cast<__bf16*>(p.O) + base;

    const int unit = gq * fsa::kWaves + wave;
    const bool active = unit < p.units_per_frame;       // uniform per wave
    const int row0 = f * T + unit * 16 * G;
    const float c = p.c;

    bf16x8 qf[G][KS];
    float shift[G], mrun[G], rs[G];
    f32x4 o[G][DB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        rs[g] = 0.f;
        mrun[g] = -INFINITY;
        shift[g] = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[g][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (active) {
        const float rsl = p.rslice[size_t(bh) * p.F + f];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int row = row0 + 16 * g + ln;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[g][ks] = *reinterpret_cast<const bf16x8*>(Qh + size_t(row) * D + 32 * ks + 8 * lj);
            shift[g] = c * (p.qnorm[size_t(bh) * p.N + row] * rsl);
        }
    }

    // ---- chunk staging: global -> registers -> LDS
    uint4 kreg[KPASS];
    uint4 vreg[4];
    const int kcol = tid % KV16;
    const int krow = tid / KV16;
    const bool vtask = tid < VTASKS;
    const int vdg = tid % KV16, vkg = tid / KV16;

    auto load_chunk = [&](int ch) {
        const int x0 = ch * BK;
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps) {
            const int x = x0 + ps * KROWS_PER_PASS + krow;
            kreg[ps] = x < sl.total
                           ? *reinterpret_cast<const uint4*>(Kh + size_t(sl.key(x)) * D + 8 * kcol)
                           : uint4{0, 0, 0, 0};
        }
        if (vtask) {
            const int x = x0 + 4 * vkg;
            if (x < sl.total) {
                const int k0 = sl.key(x);       // 4-key groups never cross a run
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vreg[i] = *reinterpret_cast<const uint4*>(Vh + size_t(k0 + i) * D + 8 * vdg);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) vreg[i] = uint4{0, 0, 0, 0};
            }
        }
    };
    auto store_chunk = [&](int st) {
        unsigned char* Ks = smem + st * STAGE;
        unsigned char* Vs = Ks + KBYTES;
#pragma unroll
        for (int ps = 0; ps < KPASS; ++ps)
            *reinterpret_cast<uint4*>(Ks + (ps * KROWS_PER_PASS + krow) * KROW + 16 * kcol) = kreg[ps];
        if (vtask) {
            const int col = 2 * (32 * (vkg >> 3) + vt_pos(vkg & 7));
            const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
            const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
            const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
            const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint2 lo = {lo_pair(v0[w], v1[w]), lo_pair(v2[w], v3[w])};
                uint2 hi = {hi_pair(v0[w], v1[w]), hi_pair(v2[w], v3[w])};
                *reinterpret_cast<uint2*>(Vs + (8 * vdg + 2 * w) * VROW + col) = lo;
                *reinterpret_cast<uint2*>(Vs + (8 * vdg + 2 * w + 1) * VROW + col) = hi;
            }
        }
    };

    load_chunk(0);
    store_chunk(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int st = ch & 1;
        const bool more = ch + 1 < nchunks;
        if (more) load_chunk(ch + 1);
        if (active) {
            const unsigned char* Ks = smem + st * STAGE;
            const unsigned char* Vs = Ks + KBYTES;
            const int nb = min(4, (sl.total - ch * BK) >> 4);     // 16-key granules
#pragma unroll
            for (int step = 0; step < 2; ++step) {
                const int kb0 = 2 * step;
                if (kb0 >= nb) break;
                const bool two = kb0 + 1 < nb;
                f32x4 sa[G], sb[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    sa[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                    sb[g] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(
                        Ks + (16 * kb0 + ln) * KROW + 64 * ks + 16 * lj);
#pragma unroll
                    for (int g = 0; g < G; ++g)
                        sa[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[g][ks], sa[g], 0, 0, 0);
                    if (two) {
                        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(
                            Ks + (16 * kb0 + 16 + ln) * KROW + 64 * ks + 16 * lj);
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            sb[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[g][ks], sb[g], 0, 0, 0);
                    }
                }
                bf16x8 pk[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float pa[4], pb[4];
                    if (fixed) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pa[i] = __builtin_amdgcn_exp2f(fmaf(sa[g][i], c, -shift[g]));
                            pb[i] = two ? __builtin_amdgcn_exp2f(fmaf(sb[g][i], c, -shift[g])) : 0.f;
                        }
                    } else {
                        float mx = fmaxf(fmaxf(sa[g][0], sa[g][1]), fmaxf(sa[g][2], sa[g][3]));
                        if (two)
                            mx = fmaxf(mx, fmaxf(fmaxf(sb[g][0], sb[g][1]), fmaxf(sb[g][2], sb[g][3])));
                        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                        const float mnew = fmaxf(mrun[g], mx);
                        const float alpha = __builtin_amdgcn_exp2f((mrun[g] - mnew) * c);
                        mrun[g] = mnew;
                        rs[g] *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db) o[g][db] *= alpha;
                        const float sh = mnew * c;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pa[i] = __builtin_amdgcn_exp2f(fmaf(sa[g][i], c, -sh));
                            pb[i] = two ? __builtin_amdgcn_exp2f(fmaf(sb[g][i], c, -sh)) : 0.f;
                        }
                    }
                    rs[g] += (pa[0] + pa[1]) + (pa[2] + pa[3]);
                    if (two) rs[g] += (pb[0] + pb[1]) + (pb[2] + pb[3]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pk[g][i] = __bf16(pa[i]);
                        pk[g][4 + i] = __bf16(pb[i]);
                    }
                }
                if (two) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 va = *reinterpret_cast<const bf16x8*>(
                            Vs + (16 * db + ln) * VROW + 64 * step + 16 * lj);
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[g], o[g][db], 0, 0, 0);
                    }
                } else {
                    // a lone 16-key granule: K = 16 products, operand slots 0-3
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const i16x4 va = *reinterpret_cast<const i16x4*>(
                            Vs + (16 * db + ln) * VROW + 64 * step + 16 * lj);
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            const bf16x4 p4 = {pk[g][0], pk[g][1], pk[g][2], pk[g][3]};
                            o[g][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                va, __builtin_bit_cast(i16x4, p4), o[g][db], 0, 0, 0);
                        }
                    }
                }
            }
        }
        if (more) store_chunk(st ^ 1);
        __syncthreads();
    }

    if (!active) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float tot = rs[g] + __shfl_xor(rs[g], 16, 64);
        tot += __shfl_xor(tot, 32, 64);
        const float inv = 1.0f / tot;
        const int row = row0 + 16 * g + ln;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            bf16x4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = __bf16(o[g][db][i] * inv);
            *reinterpret_cast<bf16x4*>(Oh + size_t(row) * D + 16 * db + 4 * lj) = out;
        }
    }
}

// fp32 route: one thread per query row, VALU arithmetic, the same slice walk
// and the same two routes. For fp32 shapes (no fp32 MFMA needed for them).
template <int D>
__global__ __launch_bounds__(64) void fwd_f32(const FwdArgs p) {
    const int64_t gid = int64_t(blockIdx.x) * 64 + threadIdx.x;
    if (gid >= int64_t(p.BH) * p.N) return;
    const int bh = int(gid / p.N), i = int(gid % p.N);
    const int T = p.T, f = i / T;
    const Slice sl = slice_of(p.tab, f, T);
    const size_t base = size_t(bh) * p.N * D;
    const bool fixed = use_fixed(p, bh);
    const float* Qh = static_cast<const float*>(p.Q) + base;
    const float* Kh = static_cast<const float*>(fixed ? p.Kc : p.K) + base;
    const float* Vh = static_cast<const float*>(p.V) + base;
    float* Oh = static_cast<float*>(p.O) + base;
    const float c = p.c;

    float q[D], o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        q[e] = Qh[size_t(i) * D + e];
        o[e] = 0.f;
    }
    const float shift = c * (p.qnorm[size_t(bh) * p.N + i] * p.rslice[size_t(bh) * p.F + f]);
    float m = -INFINITY, rs = 0.f;
    for (int x = 0; x < sl.total; ++x) {
        const int j = sl.key(x);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(q[e], Kh[size_t(j) * D + e], s);
        float w;
        if (fixed) {
            w = exp2f(fmaf(s, c, -shift));
        } else {
            if (s > m) {
                const float alpha = exp2f((m - s) * c);
                rs *= alpha;
#pragma unroll
                for (int e = 0; e < D; ++e) o[e] *= alpha;
                m = s;
            }
            w = exp2f(fmaf(s, c, -m * c));
        }
        rs += w;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(w, Vh[size_t(j) * D + e], o[e]);
    }
    const float inv = 1.0f / rs;
#pragma unroll
    for (int e = 0; e < D; ++e) Oh[size_t(i) * D + e] = o[e] * inv;
}

template <int D, int G>
void launch_bf16(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_bf16<D, G>), dim3(a.nwg), dim3(fsa::kThreads), 0, stream, a);
}

}  // namespace

namespace fsa {

fsa_status launch_forward(const fsa_plan& p, const void* Q, const void* K, const void* V,
                          void* O, const void* wsv, float scale, int32_t mode,
                          hipStream_t stream) {
    const fsa_shape& s = p.shape;
    const char* ws = static_cast<const char*>(wsv);
    FwdArgs a;
    a.Q = Q;
    a.Kc = ws + p.ws.kc;
    a.K = K;
    a.V = V;
    a.O = O;
    a.qnorm = reinterpret_cast<const float*>(ws + p.ws.qnorm);
    a.rslice = reinterpret_cast<const float*>(ws + p.ws.rslice);
    a.elig = reinterpret_cast<const uint8_t*>(ws + p.ws.elig);
    a.c = scale * kLog2e;
    a.N = s.F * s.T;
    a.T = s.T;
    a.F = s.F;
    a.BH = s.B * s.H;
    a.units_per_frame = p.forward.units_per_frame;
    a.groups_per_frame = p.forward.groups_per_frame;
    a.mode = mode;
    a.tab = p.table;
    if (s.dtype == FSA_F32) {
        const int64_t rows = int64_t(a.BH) * a.N;
        a.nwg = int32_t((rows + 63) / 64);
        if (s.d == 128)
            hipLaunchKernelGGL(fwd_f32<128>, dim3(a.nwg), dim3(64), 0, stream, a);
        else
            hipLaunchKernelGGL(fwd_f32<64>, dim3(a.nwg), dim3(64), 0, stream, a);
    } else {
        if (p.forward.workgroups > 0x7fffffffLL) {
            set_error("fsa_forward: grid of %lld workgroups too large",
                      static_cast<long long>(p.forward.workgroups));
            return FSA_ERR_UNSUPPORTED;
        }
        a.nwg = int32_t(p.forward.workgroups);
        const int G = p.forward.granules;
        if (s.d == 128) {
            switch (G) {
                case 1: launch_bf16<128, 1>(a, stream); break;
                case 2: launch_bf16<128, 2>(a, stream); break;
                case 3: launch_bf16<128, 3>(a, stream); break;
                default:
                    set_error("fsa_forward: %d granules per wave unsupported at d=128", G);
                    return FSA_ERR_UNSUPPORTED;
            }
        } else {
            switch (G) {
                case 1: launch_bf16<64, 1>(a, stream); break;
                case 2: launch_bf16<64, 2>(a, stream); break;
                case 3: launch_bf16<64, 3>(a, stream); break;
                case 4: launch_bf16<64, 4>(a, stream); break;
                default: launch_bf16<64, 5>(a, stream); break;
            }
        }
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("fsa_forward: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return FSA_OK;
}

}  // namespace fsa
