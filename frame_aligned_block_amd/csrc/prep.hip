// The producer of the attention's inputs, fused into one kernel with the
// statistics its bounds need.
//
// Source: "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
// (news.xcc.im/article/5328). "Layout Is the ABI" ¶2: the chain of small
// operations that produces attention's inputs (normalization, rotary
// embeddings, projections, head packing) is fused into one kernel that writes
// exactly the layout its consumer wants. "Unchaining the Softmax" ¶2: the
// attention's fixed max needs each query's norm and the keys' mean; this
// kernel emits both as an epilogue, so the bounds step no longer reads Q and
// reads K once instead of twice.
//
// Per token n (C = H*d channels, frame-major on an F x Hg x Wg latent grid):
//   x_hat = x * rsqrt(mean(x^2) + eps) * gamma;   y = W x_hat  (W: [3C][C]);
//   q, k, v = the three C-blocks of y, head h = channels [h*d, (h+1)*d);
//   q, k turned by the 3-D rotary embedding of the token's (t, y, x);
//   written head-packed, [B][H][N][d] bf16.
// gamma is folded into the weights once (fsa_prep_pack_weights: W' = W*gamma),
// and the row scale rsqrt(mean(x^2) + eps) is applied in the epilogue, which is
// exact: (x * s * gamma) W^T = s * (x W'^T).
//
// gfx950 design: the projection is a plain GEMM of 46,800 x 9,216 x 3,072 at
// the 720p shape. One workgroup of 8 waves per CU (two waves per SIMD)
// computes a 256-token x 256-channel tile (two heads of q, k or v) as the
// transposed product Y^T = W' X^T on v_mfma_f32_16x16x32_bf16. Each wave owns
// 64 tokens of one head (32 accumulators, 128 registers); a lane ends with 4
// consecutive channels of each 16-channel block of each of its tokens, so
// rotation pairs are in-lane and the row norm reduces like the attention's
// row sums. W' and X stream through a four-stage LDS ring of 32-channel
// chunks (4 x 32 KB) by direct-to-LDS copies issued three chunks ahead, each
// wave's share spread among its products: issuing a copy stalls the wave
// while the CU's address unit works through the queue, and the other wave on
// the SIMD keeps the matrix unit busy meanwhile. While a chunk's products run,
// the wave already reads the next chunk's operands, two after each of the
// first runs. The RMSNorm row scales come from a short pre-pass over X
// (prep_rowscale), so the GEMM loop does no vector arithmetic at all.
#include <hip/hip_runtime.h>

#include <cmath>

#include "fsa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kPrepWaves = 8;             // waves of a workgroup: two per SIMD, one workgroup per CU
constexpr int kTG = 64;                   // tokens per wave (4 granules of 16)
constexpr int kTok = fsa::kPrepTile;      // tokens per tile
constexpr int kWRows = kTok / kTG;        // wave rows of a tile
constexpr int kCh = 128;                  // output channels per wave: one head of width 128
constexpr int kCols = kPrepWaves / kWRows;    // heads per workgroup: wave columns
static_assert(kCols * kWRows == kPrepWaves, "waves tile the workgroup");
constexpr int kRows = kCols * kCh;        // W' rows of a tile
constexpr int kKC = 32;                   // input channels per LDS chunk (one k-step)
constexpr int kWSub = kRows * 64;         // a [256 rows][32 columns] chunk of W', bytes
constexpr int kXSub = kTok * 64;          // the same for X
constexpr int kStage = kWSub + kXSub;
constexpr int kStages = 4;                // LDS ring depth: copies run kStages-1 chunks ahead
constexpr int kPerCU = 1;                 // workgroups per CU
static_assert(kPerCU * (kStages * kStage + kPrepWaves * 128 * 4) <= 160 * 1024, "rings within the CU's 160 KB of LDS");
constexpr int kCopiesPerChunk = (kRows + kTok) / 16 / kPrepWaves;   // direct-to-LDS copies per wave
static_assert(kCopiesPerChunk <= kCh / 16, "one copy after each run of products");
constexpr int kMaxPairs = 64;             // channel pairs of a head (d <= 128)

struct PrepArgs {
    const void* X;        // [B][N][C] bf16
    const void* Wp;       // [3C][C] bf16, gamma folded in
    void* Q;              // [B][H][N][d] bf16
    void* K;
    void* V;
    float* qnorm;         // [B][H][N]: ||q|| of the bf16 outputs
    float* ksum;          // [B][H][tiles][d]: per-tile column sums of the bf16 keys
    const float* rscale;  // [B][N]: 1 / sqrt(mean(x^2) + eps)
    int32_t B, H, N, C, T, Wg, tiles, pairs;
    int32_t nwg;
    float eps;
    float freq_rev[kMaxPairs];   // rotation speed of each channel pair, revolutions per step
};

__device__ __forceinline__ int xcd_remap(int hw, int n) {
    const int q = n >> 3, r = n & 7;
    const int x = hw & 7, s = hw >> 3;
    return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

#define PREP_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8))

__device__ __forceinline__ void lds_copy16(unsigned lds, const void* gbase, unsigned voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff), "s"(gbase) : "memory");
}

// The copies of a wave's share of input channel chunk kc. The chunk is
// kRows/16 blocks of W' (the workgroup's output channels; rows past the last
// head repeat it, never stored), then kTok/16 blocks of X (rows past the last
// token repeat it, never stored), each 16 rows x 64 bytes; wave w takes blocks
// j = kPrepWaves * i + w, so copies 0-1 are blocks of W' and 2-3 of X. The
// 16-byte segment is swizzled by (row >> 1) & 3. Each lane's global offset
// and LDS offset are the same for every chunk (CopyPlan, computed once); the
// chunk's offset of kc * 64 bytes is uniform and rides on the scalar base, so
// issuing a copy takes no vector instruction.
struct CopyPlan {
    unsigned voff[kCopiesPerChunk];
    unsigned lds[kCopiesPerChunk];
};
static_assert(kRows / 16 == 2 * kPrepWaves && kTok / 16 == 2 * kPrepWaves && kCopiesPerChunk == 4,
              "copies 0-1 of W', 2-3 of X");

__device__ __forceinline__ CopyPlan copy_plan(int nwrows, int ntok, int C, int wave, int lane) {
    CopyPlan cp;
    const int seg = lane & 3, rr = lane >> 2;
    const unsigned col = 16 * (seg ^ ((lane >> 3) & 3));
#pragma unroll
    for (int i = 0; i < kCopiesPerChunk; ++i) {
        const int j = kPrepWaves * i + wave;
        if (i < 2) {
            const int wrow = min(16 * j + rr, nwrows - 1);
            cp.voff[i] = unsigned(wrow) * unsigned(C) * 2 + col;
            cp.lds[i] = j * 1024;
        } else {
            const int rb = j - kRows / 16;
            const int xrow = min(16 * rb + rr, ntok - 1);
            cp.voff[i] = unsigned(xrow) * unsigned(C) * 2 + col;
            cp.lds[i] = kWSub + rb * 1024;
        }
    }
    return cp;
}

__device__ __forceinline__ void issue_copy(unsigned stage, const unsigned char* Wrows,
                                           const unsigned char* Xrows, int kc, const CopyPlan& cp,
                                           int i) {
    const unsigned char* base = (i < 2 ? Wrows : Xrows) + size_t(kc) * (kKC * 2);
    lds_copy16(stage + cp.lds[i], base, cp.voff[i]);
}

// All of a wave's copies of chunk kc.
__device__ __forceinline__ void issue_chunk(unsigned stage, const unsigned char* Wrows,
                                            const unsigned char* Xrows, int kc, const CopyPlan& cp) {
#pragma unroll
    for (int i = 0; i < kCopiesPerChunk; ++i) issue_copy(stage, Wrows, Xrows, kc, cp, i);
}

// Operand i of this wave for one chunk, one 16-byte read per lane: i < G are
// its G token granules of X, the rest its head's NB channel blocks of W'.
template <int G, int NB>
__device__ __forceinline__ void load_operand(const unsigned char* S, int wr, int wc, int ka, int i,
                                             bf16x8 (&xb)[G], bf16x8 (&wa)[NB]) {
    if (i < G)
        xb[i] = *reinterpret_cast<const bf16x8*>(S + kWSub + (kTG * wr + 16 * i) * 64 + ka);
    else
        wa[i - G] = *reinterpret_cast<const bf16x8*>(S + (kCh * wc + 16 * (i - G)) * 64 + ka);
}

template <int G, int NB>
__device__ __forceinline__ void load_operands(const unsigned char* S, int wr, int wc, int ka,
                                              bf16x8 (&xb)[G], bf16x8 (&wa)[NB]) {
#pragma unroll
    for (int i = 0; i < G + NB; ++i) load_operand<G, NB>(S, wr, wc, ka, i, xb, wa);
}

// The next chunk's operands are read during the current chunk's products, two
// after each of the first kLoadRuns runs: issued all at once after the
// barrier, the 8 waves' 96 reads queue at the LDS and hold up each wave's
// first products behind its own reads (measured 3-4% slower).
constexpr int kLoadRuns = 6;
static_assert(kLoadRuns <= kCh / 16, "reads fit among the runs of products");

template <int G, int NB, typename Between>
__device__ __forceinline__ void products(const bf16x8 (&xb)[G], const bf16x8 (&wa)[NB],
                                         f32x4 (&acc)[G][NB], Between between) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
        for (int g = 0; g < G; ++g)
            acc[g][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[cb], xb[g], acc[g][cb], 0, 0, 0);
        between(cb);            // after each run of G products
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Wait until at most `later` chunks' copies of this wave are still in flight
// (loads complete in issue order), i.e. until the chunk issued just before
// them has landed. 0 <= later < kStages.
#define PREP_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
__device__ __forceinline__ void wait_chunk(int later) {
    static_assert(kStages <= 4 && kCopiesPerChunk * 3 <= 63, "vmcnt field");
    switch (later) {
        case 3: PREP_VMCNT(kCopiesPerChunk * 3); break;
        case 2: PREP_VMCNT(kCopiesPerChunk * 2); break;
        case 1: PREP_VMCNT(kCopiesPerChunk); break;
        default: PREP_VMCNT(0); break;
    }
}

template <int D>
__global__ __launch_bounds__(kPrepWaves * 64, kPerCU) void prep_qkv(const PrepArgs p) {
    static_assert(D == kCh, "one 128-channel head per wave column");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * kStage];
    __shared__ float red[kPrepWaves][D];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lj = lane >> 4;
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const int wr = uwave % kWRows, wc = uwave / kWRows;    // wave row (tokens), column (head)

    // Workgroups walk (8 token tiles) x (all head pairs) groups, so that the
    // ones an XCD runs at once share X chunks and W' chunks.
    const int L = xcd_remap(blockIdx.x, p.nwg);
    const int per_b = p.tiles * p.pairs;
    const int b = L / per_b, r0 = L % per_b;
    const int grp = r0 / (8 * p.pairs), within = r0 % (8 * p.pairs);
    const int gtiles = min(8, p.tiles - 8 * grp);
    const int pair = within / gtiles, tile = 8 * grp + within % gtiles;
    const int ncols = 3 * p.H;
    const int col0 = kCols * pair;
    const int col = min(col0 + wc, ncols - 1);              // this wave column's head
    const bool col_live = col0 + wc < ncols;                // uniform per wave
    const int part = col / p.H, h = col % p.H;               // 0 q, 1 k, 2 v
    const int tok0 = tile * kTok;
    const int ntok = min(kTok, p.N - tok0);

    const unsigned char* Wrows = static_cast<const unsigned char*>(p.Wp) + size_t(col0) * D * p.C * 2;
    const int nwrows = min(kRows, (ncols - col0) * D);
    const unsigned char* Xrows = static_cast<const unsigned char*>(p.X) +
                                 (size_t(b) * p.N + tok0) * p.C * 2;
    const int nchunks = p.C / kKC;
    const unsigned smem_lds = unsigned(uintptr_t((lds_void*)smem));

    constexpr int G = kTG / 16, NB = D / 16;
    f32x4 acc[G][NB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[g][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ka = ln * 64 + 16 * (lj ^ ((ln >> 1) & 3));    // this lane's 16 bytes of a 16-row block
    const CopyPlan cp = copy_plan(nwrows, ntok, p.C, uwave, lane);
    // Chunk c lives in stage c % kStages. The ring starts full.
    for (int c = 0; c < kStages && c < nchunks; ++c)
        issue_chunk(smem_lds + c * kStage, Wrows, Xrows, c, cp);
    wait_chunk(min(kStages, nchunks) - 1);               // chunk 0 has landed
    __builtin_amdgcn_s_barrier();
    bf16x8 xb[2][G], wa[2][NB];
    load_operands<G, NB>(smem, wr, wc, ka, xb[0], wa[0]);
    // One chunk: once chunk k+1 has landed and every wave holds its chunk-k
    // operands, chunk k's stage takes chunk k + kStages; then the wave reads
    // chunk k+1's operands while chunk k's products run. Two chunks per trip,
    // so each operand set keeps its registers. In the steady state two later
    // chunks' copies of this wave may still be in flight; near the end the
    // wave waits for all of them.
    auto step = [&](int k, int u, bool steady) {
        const bool more = steady || k + 1 < nchunks;
        if (more) {
            if (steady) PREP_VMCNT(kCopiesPerChunk * (kStages - 2));
            else PREP_VMCNT(0);
            __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4));   // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
        }
        // Keep the products after the barrier (the compiler would otherwise
        // hoist them above it), read chunk k+1's operands among them, and
        // spread this wave's copies of chunk k + kStages among them too: a
        // wave stalls while the CU's address unit works through its copies,
        // and the other wave on the SIMD keeps the matrix unit busy meanwhile.
        __builtin_amdgcn_sched_barrier(0);
        const bool copies = steady || (k + 1 < nchunks && k + kStages < nchunks);
        const unsigned stage = smem_lds + (k % kStages) * kStage;
        const unsigned char* next = smem + ((k + 1) % kStages) * kStage;
        products<G, NB>(xb[u], wa[u], acc, [&](int cb) {
            if (more && cb < kLoadRuns) {
#pragma unroll
                for (int i = cb * (G + NB) / kLoadRuns; i < (cb + 1) * (G + NB) / kLoadRuns; ++i)
                    load_operand<G, NB>(next, wr, wc, ka, i, xb[u ^ 1], wa[u ^ 1]);
            }
            if (copies && cb < kCopiesPerChunk)
                issue_copy(stage, Wrows, Xrows, k + kStages, cp, cb);
        });
    };
    // Steady trips have no branch inside: chunk k+1 exists, chunks k+2 and
    // k+3 were issued after it, and chunk k + kStages exists (k + 1 + kStages
    // < nchunks for both steps of the trip).
    const int steady_end = max(0, (nchunks - kStages) & ~1);
    int kc = 0;
    for (; kc < steady_end; kc += 2) {
        step(kc, 0, true);
        step(kc + 1, 1, true);
    }
    for (; kc < nchunks; kc += 2) {
        step(kc, 0, false);
        if (kc + 1 < nchunks) step(kc + 1, 1, false);
    }
    PREP_WAIT_VMCNT0();

    // ---- epilogue: row scale, rotation, rounding, statistics, store
    // Each wave stages its 64 x 128 bf16 output tile in its own 16 KB of the
    // ring (free once every wave has passed the barrier below) and stores it
    // back as whole 256-byte rows, 16 bytes a lane: half the store
    // instructions of storing each lane's 4 channels, and whole cache lines.
    // In row r, 16-byte segment s sits at s ^ (r & 7) and its two 8-byte
    // halves trade places when r & 8, so that the 16 rows one write
    // instruction touches fill 128 distinct bytes of banks and each row read
    // takes whole lines.
    static_assert(kPrepWaves * kTG * kCh * 2 <= kStages * kStage, "staging fits the ring");
    __syncthreads();                                     // no wave reads the ring any more
    const unsigned stage_out = smem_lds + uwave * (kTG * kCh * 2);
    const bool rotate = part < 2;
    __bf16* out = static_cast<__bf16*>(part == 0 ? p.Q : part == 1 ? p.K : p.V) +
                  (size_t(b) * p.H + h) * p.N * D;
    float csum[NB][4];                       // key column sums over this lane's tokens
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) csum[cb][e] = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int tl = kTG * wr + 16 * g + ln;           // token within the tile
        const bool live = col_live && tl < ntok;
        const int n = tok0 + min(tl, ntok - 1);
        const float rs = p.rscale[size_t(b) * p.N + n];
        const int f = n / p.T, pin = n % p.T;
        const float pos[3] = {float(f), float(pin / p.Wg), float(pin % p.Wg)};
        float qq = 0.f;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = acc[g][cb][e] * rs;
            if (rotate) {
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const int c = 16 * cb + 4 * lj + e;          // even channel of the pair
                    const int band = c < D / 4 ? 0 : (c < D / 4 + 3 * D / 8 ? 1 : 2);
                    const float rev = pos[band] * p.freq_rev[c >> 1];
                    const float cs = __builtin_amdgcn_cosf(rev - floorf(rev));
                    const float sn = __builtin_amdgcn_sinf(rev - floorf(rev));
                    const float a = y[e], bb = y[e + 1];
                    y[e] = a * cs - bb * sn;
                    y[e + 1] = a * sn + bb * cs;
                }
            }
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = __bf16(y[e]);
            if (part == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) qq = fmaf(float(o4[e]), float(o4[e]), qq);
            } else if (part == 1 && live) {
#pragma unroll
                for (int e = 0; e < 4; ++e) csum[cb][e] += float(o4[e]);
            }
            {
                const int r = 16 * g + ln;                   // row of the wave's tile
                const unsigned seg = unsigned(2 * cb + (lj >> 1)) ^ unsigned(r & 7);
                const unsigned half = unsigned(lj & 1) ^ unsigned((r >> 3) & 1);
                *(lds_bf16x4*)(stage_out + r * (kCh * 2) + seg * 16 + half * 8) = o4;
            }
        }
        if (part == 0) {
            qq += __shfl_xor(qq, 16, 64);
            qq += __shfl_xor(qq, 32, 64);
            if (live && lj == 0) p.qnorm[(size_t(b) * p.H + h) * p.N + n] = sqrtf(qq);
        }
    }
    // the staged tile, 4 rows per read: lane l takes row 4i + l/16, segment l%16
    if (col_live) {
#pragma unroll
        for (int i = 0; i < kTG / 4; ++i) {
            const int r = 4 * i + (lane >> 4), sg = lane & 15;
            const int tl = kTG * wr + r;
            bf16x8 v = *(const lds_bf16x8*)(stage_out + r * (kCh * 2) + ((sg ^ (r & 7)) * 16));
            if ((r >> 3) & 1) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
            if (tl < ntok) *reinterpret_cast<bf16x8*>(out + size_t(tok0 + tl) * D + 8 * sg) = v;
        }
    }
    // key column sums: over the 16 tokens of each lane group, then the 2 wave
    // rows of the column, in order (every wave passes the same barrier)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = csum[cb][e];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            if (ln == 0) red[uwave][16 * cb + 4 * lj + e] = v;
        }
    __syncthreads();
    if (part == 1 && col_live && wr == 0) {
        for (int c = lane; c < D; c += 64) {
            float s = red[kWRows * wc][c];
#pragma unroll
            for (int r = 1; r < kWRows; ++r) s += red[kWRows * wc + r][c];
            p.ksum[((size_t(b) * p.H + h) * p.tiles + tile) * D + c] = s;
        }
    }
}

// RMSNorm row scale of every token: 1 / sqrt(mean_c x_c^2 + eps), fp32 from
// the bf16 tokens; 16 lanes per token, 16 tokens per workgroup.
__global__ __launch_bounds__(256) void prep_rowscale(const __bf16* __restrict__ X,
                                                     float* __restrict__ rscale, int64_t rows,
                                                     int C, float eps) {
    const int64_t row = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    if (row >= rows) return;                 // whole 16-lane groups: the shuffles stay in-group
    const __bf16* x = X + row * C;
    float s = 0.f;
    int c = 8 * l;
    for (; c + 3 * 128 < C; c += 4 * 128) {            // four loads a trip, issued together
        bf16x8 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const bf16x8*>(x + c + u * 128);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(float(v[u][e]), float(v[u][e]), s);
    }
    for (; c < C; c += 128) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + c);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(float(v[e]), float(v[e]), s);
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 16);
    if (l == 0) rscale[row] = 1.0f / sqrtf(s / float(C) + eps);
}

// W' = W * gamma (per input channel), rounded to bf16.
__global__ __launch_bounds__(256) void prep_fold(const __bf16* __restrict__ W,
                                                 const float* __restrict__ gamma,
                                                 __bf16* __restrict__ Wp, int64_t n, int C) {
    const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
    if (i >= n) return;
    const bf16x8 w = *reinterpret_cast<const bf16x8*>(W + i);
    bf16x8 o;
    const int c0 = int(i % C);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = __bf16(float(w[e]) * gamma[c0 + e]);
    *reinterpret_cast<bf16x8*>(Wp + i) = o;
}

// The key mean from the producer's per-tile column sums, in tile order.
template <int D>
__global__ __launch_bounds__(256) void prep_mean(const float* __restrict__ ksum,
                                                 float* __restrict__ mu, int tiles, int N) {
    const int bh = blockIdx.x, t = threadIdx.x;
    if (t >= D) return;
    float s = 0.f;
    const float* col = ksum + size_t(bh) * tiles * D + t;
#pragma unroll 8
    for (int i = 0; i < tiles; ++i) s += col[size_t(i) * D];
    mu[size_t(bh) * D + t] = s / float(N);
}

// Per part (at most 256 rows of one frame): the largest ||k_j - mu|| from the
// keys, the largest ||q_i|| from the producer's row norms, and the part's key
// column sums (for the slices' mean keys; the producer's own sums are per
// 256-token tile, which may straddle frames).
template <int D>
__global__ __launch_bounds__(256) void prep_radius(const __bf16* __restrict__ K,
                                                   const float* __restrict__ mu,
                                                   const float* __restrict__ qnorm,
                                                   float* __restrict__ partmax,
                                                   float* __restrict__ partqmax,
                                                   float* __restrict__ colsum, int N, int T,
                                                   int rows_per_part, int ppf, int nparts) {
    constexpr int LPR = D / 8;
    constexpr int RPI = 256 / LPR;
    __shared__ float red[RPI], qred[256];
    __shared__ float cred[RPI][D];
    const int part = blockIdx.x, bh = blockIdx.y;
    const int frame = part / ppf, sub = part % ppf;
    const int begin = frame * T + sub * rows_per_part;
    const int end = min(frame * T + T, begin + rows_per_part);
    const int lane = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
    const __bf16* Kh = K + size_t(bh) * N * D;
    float m[8], acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        m[e] = mu[size_t(bh) * D + lane * 8 + e];
        acc[e] = 0.f;
    }
    float best = 0.f;
    auto krow = [&](const bf16x8& k) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ke = float(k[e]);
            acc[e] += ke;
            const float c = ke - m[e];
            s = fmaf(c, c, s);
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
        best = fmaxf(best, sqrtf(s));
    };
    int r = begin + r0;
    for (; r + 3 * RPI < end; r += 4 * RPI) {          // four rows a trip, loads together
        bf16x8 kk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) kk[u] = *reinterpret_cast<const bf16x8*>(Kh + size_t(r + u * RPI) * D + lane * 8);
#pragma unroll
        for (int u = 0; u < 4; ++u) krow(kk[u]);
    }
    for (; r < end; r += RPI) {
        const bf16x8 k = *reinterpret_cast<const bf16x8*>(Kh + size_t(r) * D + lane * 8);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ke = float(k[e]);
            acc[e] += ke;
            const float c = ke - m[e];
            s = fmaf(c, c, s);
        }
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
        best = fmaxf(best, sqrtf(s));
    }
    float qb = 0.f;
    for (int r = begin + int(threadIdx.x); r < end; r += 256)
        qb = fmaxf(qb, qnorm[size_t(bh) * N + r]);
    if (lane == 0) red[r0] = best;
    qred[threadIdx.x] = qb;
#pragma unroll
    for (int e = 0; e < 8; ++e) cred[r0][lane * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float cs = 0.f;
        for (int i = 0; i < RPI; ++i) cs += cred[i][threadIdx.x];
        colsum[(size_t(bh) * nparts + part) * D + threadIdx.x] = cs;
    }
    if (threadIdx.x == D) {
        float b = 0.f, q = 0.f;
        for (int i = 0; i < RPI; ++i) b = fmaxf(b, red[i]);
        for (int i = 0; i < 256; ++i) q = fmaxf(q, qred[i]);
        partmax[size_t(bh) * nparts + part] = b;
        partqmax[size_t(bh) * nparts + part] = q;
    }
}

}  // namespace

namespace fsa {

fsa_status launch_prep_fold(const void* W, const float* gamma, void* Wp, int32_t C,
                            hipStream_t stream) {
    const int64_t n = int64_t(3) * C * C;
    const int64_t blocks = (n / 8 + 255) / 256;
    hipLaunchKernelGGL(prep_fold, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<const __bf16*>(W), gamma, static_cast<__bf16*>(Wp), n, C);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("fsa_prep_pack_weights: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return FSA_OK;
}

fsa_status launch_prep(const fsa_plan& p, int32_t Wg, const void* X, const void* Wp, void* Q,
                       void* K, void* V, void* wsv, hipStream_t stream) {
    const fsa_shape& s = p.shape;
    char* ws = static_cast<char*>(wsv);
    PrepArgs a;
    a.X = X;
    a.Wp = Wp;
    a.Q = Q;
    a.K = K;
    a.V = V;
    a.qnorm = reinterpret_cast<float*>(ws + p.ws.qnorm);
    a.ksum = reinterpret_cast<float*>(ws + p.prep_ksum);
    a.rscale = reinterpret_cast<const float*>(ws + p.prep_rscale);
    a.B = s.B;
    a.H = s.H;
    a.N = s.F * s.T;
    a.C = s.H * s.d;
    a.T = s.T;
    a.Wg = Wg;
    a.tiles = (a.N + kTok - 1) / kTok;
    a.pairs = (3 * s.H + kCols - 1) / kCols;
    a.eps = kPrepEps;
    // pair i of band b (n_b channels): 10000^(-2i/n_b) radians per step
    const int bands[3] = {s.d / 4, 3 * s.d / 8, 3 * s.d / 8};
    int pi = 0;
    for (int bnd = 0; bnd < 3; ++bnd)
        for (int i = 0; i < bands[bnd] / 2; ++i)
            a.freq_rev[pi++] = float(std::pow(double(kPrepBase), -2.0 * i / bands[bnd]) /
                                     (2.0 * 3.14159265358979323846));
    for (; pi < kMaxPairs; ++pi) a.freq_rev[pi] = 0.f;
    const int64_t nwg = int64_t(s.B) * a.tiles * a.pairs;
    if (nwg > 0x7fffffffLL) {
        set_error("fsa_prep: grid too large");
        return FSA_ERR_UNSUPPORTED;
    }
    a.nwg = int32_t(nwg);
    const int64_t rows = int64_t(s.B) * a.N;
    hipLaunchKernelGGL(prep_rowscale, dim3(unsigned((rows + 15) / 16)), dim3(256), 0, stream,
                       static_cast<const __bf16*>(X), reinterpret_cast<float*>(ws + p.prep_rscale),
                       rows, a.C, a.eps);
    hipLaunchKernelGGL((prep_qkv<128>), dim3(a.nwg), dim3(kPrepWaves * 64), 0, stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("fsa_prep: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return FSA_OK;
}

fsa_status launch_bounds_after_prep(const fsa_plan& p, const void* K, void* wsv, float scale,
                                    hipStream_t stream) {
    const fsa_shape& s = p.shape;
    char* ws = static_cast<char*>(wsv);
    const int N = s.F * s.T, BH = s.B * s.H;
    const int tiles = (N + kTok - 1) / kTok;
    const Parts& q = p.bounds.q;
    float* mu = reinterpret_cast<float*>(ws + p.ws.mu);
    float* partmax = reinterpret_cast<float*>(ws + p.bounds.partmax);
    float* partqmax = reinterpret_cast<float*>(ws + p.bounds.partqmax);
    hipLaunchKernelGGL((prep_mean<128>), dim3(BH), dim3(256), 0, stream,
                       reinterpret_cast<const float*>(ws + p.prep_ksum), mu, tiles, N);
    hipLaunchKernelGGL((prep_radius<128>), dim3(q.count(), BH), dim3(256), 0, stream,
                       static_cast<const __bf16*>(K), mu,
                       reinterpret_cast<const float*>(ws + p.ws.qnorm), partmax, partqmax,
                       reinterpret_cast<float*>(ws + p.bounds.colsum), N, s.T,
                       q.rows_per_part, q.per_frame, q.count());
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        set_error("fsa_bounds_after_prep: launch failed: %s", hipGetErrorString(err));
        return FSA_ERR_HIP;
    }
    return launch_bounds_finalize(p, ws, scale, stream);
}

}  // namespace fsa
