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
//  * Each wave owns 16*G consecutive query rows of one frame (a row unit); the
//    waves of a workgroup own consecutive row units of the same frame, so they
//    share one key slice. The slice is at most two contiguous token runs (the
//    clipped window, and the reference frame when it lies outside it), read
//    from a per-frame table passed as a kernel argument. The runs are walked
//    as one sequence in chunks of 64 keys; only the very last chunk can be
//    shorter (16, 32 or 48 keys, a whole number of 16-key granules, so still
//    no partial block).
//  * Two workgroup geometries, recorded in the plan:
//    - 4 waves (128 rows), two workgroups per CU, the plan's choice: K and V
//      chunks stream into a 2-stage LDS ring by direct-to-LDS copies, shared
//      by the 4 waves, with one barrier per chunk;
//    - 8 waves (256 rows), one workgroup per CU, on request: a 4-stage ring
//      with one barrier per pair of chunks, each chunk copied once for twice
//      the rows; the copies of the pair after next are issued right after
//      each barrier.
//    In both, a frame's last workgroup, when left with a single row unit,
//    splits the key chunks among its waves instead (attend_split,
//    attend_split8); the V^T operand of P.V is read transposed out of
//    row-major V (ds_read_b64_tr_b16), and two waves share each SIMD.
//  * Every route scores K as given. The fixed route's shift for row i is its
//    bound on the centred scores, scale ||q_i|| R_S, plus scale q_i.mu:
//    centring moves every score of the row by that amount, so the softmax is
//    the same and no centred copy of K is ever stored. A fixed wave whose rows
//    keep c ||q_i|| R_S within FSA_SCALED_LIMIT takes the scaled fixed route:
//    the scale rides in its query fragments and the shift is the products'
//    starting value, so each probability is a single exp2 of a product.
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
    const void* K;
    const void* V;
    void* O;
    const float* mu;            // key mean per (batch, head)
    const float* qnorm;
    const float* rslice;
    const uint8_t* elig;        // per (batch, head)
    const uint8_t* eligf;       // per (batch, head, frame)
    const float* dslice;        // slice mean key minus mu, per (batch, head, frame)
    unsigned* pmax;             // largest fixed-route probability (float bits), kernels with PMAX
    float c;                    // scale * log2(e)
    int32_t N, T, F, BH;
    int32_t NK;                 // key (and value) tokens per (batch, head)
    int32_t KT;                 // tokens per key frame: the run table's unit
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

// Query frame f's key slice, in tokens: the run table counts key frames of KT
// tokens (the chunk's frames, or the whole reference set for cross-attention).
__device__ __forceinline__ Slice slice_of(const FrameTable& t, int f, int KT) {
    const uint32_t run = t.runs[f];
    Slice s;
    s.s0 = int(run & 0xff) * KT;
    s.n0 = int((run >> 8) & 0xff) * KT;
    s.s1 = int((run >> 16) & 0xff) * KT;
    s.total = s.n0 + int(run >> 24) * KT;
    return s;
}

// The route of a (batch*head, frame) pair from the flags of fsa_bounds. Under
// AUTO_ROWS the kernels decide from the rows themselves (row_gap_ok).
__device__ __forceinline__ bool use_fixed(const FwdArgs& p, int bh, int f) {
    if (p.mode == FSA_MODE_FIXED_ONLY) return true;
    if (p.mode == FSA_MODE_ONLINE_ONLY || p.mode == FSA_MODE_AUTO_ROWS) return false;
    if (p.mode == FSA_MODE_AUTO_FRAME) return p.eligf[size_t(bh) * p.F + f] != 0;
    return p.elig[bh] != 0;
}

// Whether a gap bound, kept in units of 1/scale (||q_i|| R_S - q_i.dslice),
// is within FSA_GAP_LIMIT once scaled: c = scale * log2(e).
__device__ __forceinline__ bool row_gap_ok(float g, float c) {
    return g * c <= FSA_GAP_LIMIT * kLog2e;
}

// Whether the (batch*head, frame) pairs of this launch take different routes
// (then their costs differ by the online route's ~1.3x). Every wave reads all
// the flags itself (no LDS, no barrier) and every wave of every workgroup
// reaches the same answer; launches past kMixScan pairs are treated as
// uniform.
constexpr int kMixScan = 4096;

__device__ __forceinline__ bool routes_mixed(const FwdArgs& p) {
    const uint8_t* fl;
    int n;
    if (p.mode == FSA_MODE_AUTO) {
        fl = p.elig;
        n = p.BH;
    } else if (p.mode == FSA_MODE_AUTO_FRAME || p.mode == FSA_MODE_AUTO_ROWS) {
        // (AUTO_ROWS: the per-frame flags stand in for routes decided later)
        fl = p.eligf;
        n = p.BH * p.F;
    } else {
        return false;
    }
    if (n > kMixScan) return false;
    const uint8_t first = fl[0];
    bool diff = false;
    for (int i = threadIdx.x & 63; i < n; i += 64) diff |= fl[i] != first;
    return __builtin_amdgcn_ballot_w64(diff) != 0;
}

// The pair of the ti-th place in the launch order. Uniform launches walk the
// pairs in order, so each XCD (a contiguous range of places) holds whole heads
// with their frames side by side and shares their key slices in its L2. Mixed
// launches deal the pairs out x, x+8, x+16, ... for x = 0..7, so each XCD gets
// its share of the online pairs. A bijection on [0, BH*F).
__device__ __forceinline__ int pair_at(const FwdArgs& p, int ti, bool mixed) {
    if (!mixed) return ti;
    const int P = p.BH * p.F, q8 = P >> 3, r8 = P & 7;
    if (ti < r8 * (q8 + 1)) return ti / (q8 + 1) + 8 * (ti % (q8 + 1));
    const int j = ti - r8 * (q8 + 1);
    return r8 + j / q8 + 8 * (j % q8);            // here q8 >= 1
}

// ---------------------------------------------------------------- bf16 route

constexpr int kBK = 64;                 // keys per LDS chunk

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// LDS tiles. A chunk's K (and V) tile is D/32 column sub-tiles of 64 rows x
// 64 bytes (32 columns each), so every read address is a per-lane constant
// plus an immediate. Small XOR swizzles keep each read pattern on distinct
// banks (64 banks x 4 bytes):
//  * K (read 16 rows at one 16-byte segment): segment ^= (row >> 1) & 3
//    (chosen by measuring SQ_LDS_BANK_CONFLICT over candidate swizzles);
//  * V (read transposed, 4 rows x 32 bytes per 16 lanes): 32-byte half
//    ^= (row >> 2) & 1.
// A tile is copied as 1 KB blocks of 16 rows x 64 bytes: block j is sub-tile
// j / RB, rows 16 (j % RB) .. +15.
template <int D>
struct Geo {
    static constexpr int KS = D / 32;                  // k-steps of S^T over d = sub-tiles
    static constexpr int DB = D / 16;                  // 16-wide column blocks of O^T
    static constexpr int SUB = kBK * 64;               // one 64 x 64-byte sub-tile
    static constexpr int TILE = KS * SUB;              // one K (or V) chunk
    static constexpr int STAGE = 2 * TILE;             // K tile, then V tile
    static constexpr int RB = kBK / 16;                // 16-row blocks per sub-tile
    static constexpr int BLOCKS = KS * RB;             // 1 KB blocks per tile
};

// vmcnt(n) with no wait on the other counters (gfx9 encoding).
#define FSA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// One 16-byte-per-lane direct global -> LDS copy: 64 lanes fill 1 KB of LDS
// at `lds` (wave-uniform) from gbase + voff. Written as inline assembly on
// purpose: the compiler's wait-count pass otherwise assumes such a copy may
// alias every later LDS read and stalls each chunk on vmcnt(0) until the copy
// issued for three chunks ahead has landed. Completion is tracked explicitly
// (FSA_WAIT_VMCNT) before the barrier that publishes a chunk. M0 is a
// reserved register the compiler never keeps values in.
__device__ __forceinline__ void lds_copy16(unsigned lds, const void* gbase, unsigned voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds), "v"(voff), "s"(gbase) : "memory");
}

// Asynchronous global -> LDS copies of chunk ch of the slice walk (K and V
// straight into the stage, no registers). A workgroup of W waves numbers the
// tile's 1 KB blocks j = W i + w for the block groups i < BLOCKS / W and its
// waves w; W is a multiple of RB, so the blocks of w always hold the same 16
// rows: lane l carries row 16 (w % RB) + l/4, 16-byte segment l%4. Positions
// past the slice are clamped to its last key: harmless duplicates that are
// never read. issue_group issues group i of the blocks of w: one K and one V
// copy.
template <int D, int W>
__device__ __forceinline__ void issue_group(unsigned stage_lds, const Slice& sl, const __bf16* Kh,
                                            const __bf16* Vh, int ch, int wave, int lane, int i) {
    using GG = Geo<D>;
    static_assert(W % GG::RB == 0 && GG::BLOCKS % W == 0, "waves tile the blocks");
    const int row = 16 * (wave % GG::RB) + (lane >> 2);
    const unsigned rowoff = unsigned(sl.key(min(ch * kBK + row, sl.total - 1))) * (2 * D);
    const int seg = lane & 3;
    const unsigned koff = rowoff + 16 * (seg ^ ((lane >> 3) & 3));     // (row >> 1) & 3
    const unsigned voff = rowoff + 16 * (seg ^ (((lane >> 4) & 1) << 1));
    const int j = i * W + wave;
    const int t = j / GG::RB;                          // sub-tile = 32-column block
    const unsigned dst = stage_lds + t * GG::SUB + (j % GG::RB) * 1024;
    lds_copy16(dst, reinterpret_cast<const unsigned char*>(Kh) + 64 * t, koff);
    lds_copy16(dst + GG::TILE, reinterpret_cast<const unsigned char*>(Vh) + 64 * t, voff);
}

// 4-wave workgroups: a whole chunk's copies, issued by the first two waves
// (wave w < 2 also issues the groups of wave w + 2). A wave that issues
// copies stalls while the CU's address path takes them; two copying waves
// measured 1.3-2.2% faster than all four (the others start their next step
// at once) and faster than one (too long a stall).
template <int D>
__device__ __forceinline__ void issue_chunk4(unsigned stage_lds, const Slice& sl, const __bf16* Kh,
                                             const __bf16* Vh, int ch, int wave, int lane) {
    if (wave >= 2) return;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < Geo<D>::BLOCKS / 4; ++i)
            issue_group<D, 4>(stage_lds, sl, Kh, Vh, ch, wave + 2 * r, lane, i);
}

// 8-wave workgroups: waves 0-3 (one per SIMD) issue the whole chunk, wave w
// also the groups of wave w + 4. Right after a barrier the copying waves stall
// while the CU's address path takes their copies and waves 4-7 run ahead,
// which puts the two waves of each SIMD out of phase again (the barrier had
// lined them up): measured 2.6-3.6% faster than all 8 waves copying.
template <int D>
__device__ __forceinline__ void issue_chunk8(unsigned stage_lds, const Slice& sl, const __bf16* Kh,
                                             const __bf16* Vh, int ch, int wave, int lane) {
    if (wave >= 4) return;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < Geo<D>::BLOCKS / 8; ++i)
            issue_group<D, 8>(stage_lds, sl, Kh, Vh, ch, wave + 4 * r, lane, i);
}

// Per-lane LDS byte offsets (constant for the whole walk).
struct LaneAddr {
    int k;        // K read: row ln, segment lj (swizzled)
    int v0, v1;   // V transposed read, even / odd column block
};

__device__ __forceinline__ LaneAddr lane_addr(int ln, int lj) {
    LaneAddr a;
    a.k = ln * 64 + 16 * (lj ^ ((ln >> 1) & 3));
    const int vbase = (4 * lj + (ln >> 2)) * 64 + 8 * (ln & 3);
    a.v0 = vbase + 32 * (lj & 1);
    a.v1 = vbase + 32 * ((lj & 1) ^ 1);
    return a;
}

// S^T for the 32 keys at chunk-local key koff (0 or 32): s[0] = first 16 keys,
// s[1] = next 16; the lane holds query ln of each granule and keys 4lj..4lj+3.
// The products accumulate onto s0 (per granule): zero, or on the scaled fixed
// route minus the row's shift (its query fragments then carry the scale), so
// that the scores come out as the exponents themselves.
template <int D, int G, int NB>
__device__ __forceinline__ void scores(const unsigned char* Ks, int koff,
                                       const bf16x8 (&qf)[G][D / 32], const f32x4 (&s0)[G],
                                       f32x4 (&s)[2][G], const LaneAddr& la) {
    using GG = Geo<D>;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int g = 0; g < G; ++g) s[b][g] = s0[g];
#pragma unroll
    for (int ks = 0; ks < GG::KS; ++ks) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                Ks + ks * GG::SUB + (koff + 16 * b) * 64 + la.k);
#pragma unroll
            for (int g = 0; g < G; ++g)
                s[b][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[g][ks], s[b][g], 0, 0, 0);
        }
    }
}

// V^T operand for column block db and key block b of the 32 keys at koff:
// keys 4lj..4lj+3 (+16b) of column 16db+ln, read transposed out of row-major
// V (each lane fetches 4 columns of one key row).
template <int D>
__device__ __forceinline__ bf16x4 v_operand(const unsigned char* Vs, int koff, int b, int db,
                                            const LaneAddr& la) {
    using GG = Geo<D>;
    const unsigned char* a = Vs + (db >> 1) * GG::SUB + (koff + 16 * b) * 64 + ((db & 1) ? la.v1 : la.v0);
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)a);
#else
    (void)a;
    return bf16x4{};
#endif
}

// Row sum of packed bf16 probabilities: two terms per v_dot2 (fp32 accumulate).
__device__ __forceinline__ float sum_pairs(const bf16x2* pp, int n, float acc) {
    const bf16x2 one = {__bf16(1.0f), __bf16(1.0f)};
#pragma unroll
    for (int i = 0; i < n; ++i) acc = __builtin_amdgcn_fdot2_f32_bf16(pp[i], one, acc, false);
    return acc;
}

// Routes of the slice walks (template parameter R).
constexpr int kOnline = 0;       // running reference max
constexpr int kFixed = 1;        // shift fixed at the row's Cauchy-Schwarz bound
constexpr int kFixedScaled = 2;  // kFixed on scaled query fragments, the shift in s0
constexpr int kPmax = 4;         // flag on a fixed route: keep each row's largest p in m
__host__ __device__ constexpr bool scaled_route(int r) { return (r & 3) == kFixedScaled; }
__host__ __device__ constexpr bool pmax_route(int r) { return (r & kPmax) != 0; }

// Probabilities of NK scores of one granule-row. Fixed route: the shift is
// the row's Cauchy-Schwarz bound (scale folded in, log2 units); on the scaled
// fixed route the scores already hold the exponents, so a probability is one
// exp2. With kPmax the largest probability formed (before rounding to bf16)
// is kept in m, which the fixed routes do not use otherwise. Online route: a
// running reference max, moved (with the accumulator and row sum rescaled)
// only when a step's max exceeds it by more than kLazyLog2 in log2 units, and
// only in the steps where some row of the wave needs it; until then the
// row's probabilities may reach 2^kLazyLog2, which bf16 and the fp32 sums
// hold as precisely.
constexpr float kLazyLog2 = 8.f;

template <int D, int G, int R, int NK>
__device__ __forceinline__ void probs(const f32x4* sv, int g, float c, const float (&shift)[G],
                                      float (&m)[G], float (&rs)[G], f32x4 (&o)[G][D / 16],
                                      float (&p)[NK]) {
    if (R != kOnline) {
        if (scaled_route(R)) {
#pragma unroll
            for (int i = 0; i < NK; ++i) p[i] = __builtin_amdgcn_exp2f(sv[i >> 2][i & 3]);
        } else {
#pragma unroll
            for (int i = 0; i < NK; ++i)
                p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i >> 2][i & 3], c, -shift[g]));
        }
        if (pmax_route(R)) {
#pragma unroll
            for (int i = 0; i < NK; ++i) m[g] = fmaxf(m[g], p[i]);
        }
    } else {
        float mx = sv[0][0];
#pragma unroll
        for (int i = 1; i < NK; ++i) mx = fmaxf(mx, sv[i >> 2][i & 3]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const bool grow = (mx - m[g]) * c > kLazyLog2;          // always at the first step
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {           // uniform
            const float mnew = grow ? mx : m[g];
            const float alpha = __builtin_amdgcn_exp2f((m[g] - mnew) * c);
            m[g] = mnew;
            rs[g] *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db) o[g][db] *= alpha;
        }
        const float sh = m[g] * c;
#pragma unroll
        for (int i = 0; i < NK; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i >> 2][i & 3], c, -sh));
    }
}

// V^T operands of the 32 keys at koff for all D/16 column blocks: the two
// 16-key halves form the two k-groups of the 16x16x32 B operand.
template <int D>
__device__ __forceinline__ void load_v(const unsigned char* Vs, int koff, bf16x8 (&va)[D / 16],
                                       const LaneAddr& la) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        const bf16x4 v0 = v_operand<D>(Vs, koff, 0, db, la);
        const bf16x4 v1 = v_operand<D>(Vs, koff, 1, db, la);
        va[db] = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    }
}

// Softmax of one 32-key step (NB = 2) or of the lone 16-key granule (NB = 1)
// into packed bf16 probabilities, the B operand of O^T += V^T P^T. The row
// sum adds the bf16-rounded probabilities, the values the product consumes.
template <int D, int G, int R, int NB>
__device__ __forceinline__ void softmax(const f32x4 (&s)[2][G], float c, const float (&shift)[G],
                                        float (&m)[G], float (&rs)[G], f32x4 (&o)[G][D / 16],
                                        bf16x2 (&pk)[G][2 * NB]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const f32x4 sv[2] = {s[0][g], s[1][g]};
        float p[4 * NB];
        probs<D, G, R, 4 * NB>(sv, g, c, shift, m, rs, o, p);
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) pk[g][i] = bf16x2{__bf16(p[2 * i]), __bf16(p[2 * i + 1])};
        rs[g] = sum_pairs(pk[g], 2 * NB, rs[g]);
    }
    // Keep the row sums in this step: the compiler otherwise sinks some of the
    // additions past the next barrier and its copy branch, where the packed
    // pairs are gone, and packs those pairs a second time (4 conversions and
    // 2 permutes per 64 keys; 1.6% of the 720p forward).
#pragma unroll
    for (int g = 0; g < G; ++g) asm volatile("" :: "v"(rs[g]));
}

// K operands of the 32 keys at koff: 16 rows per 16-key block, all D/32
// k-steps of the S^T product.
template <int D>
__device__ __forceinline__ void load_k(const unsigned char* Ks, int koff, bf16x8 (&ka)[D / 32][2],
                                       const LaneAddr& la) {
    using GG = Geo<D>;
#pragma unroll
    for (int ks = 0; ks < GG::KS; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            ka[ks][b] = *reinterpret_cast<const bf16x8*>(Ks + ks * GG::SUB + (koff + 16 * b) * 64 + la.k);
}

template <int G>
__device__ __forceinline__ bf16x8 pack_p(const bf16x2 (&pk)[G][4], int g) {
    return bf16x8{pk[g][0][0], pk[g][0][1], pk[g][1][0], pk[g][1][1],
                  pk[g][2][0], pk[g][2][1], pk[g][3][0], pk[g][3][1]};
}

// The matrix phase of a step: S^T of the next 32 keys (sn, from their K
// operands ka) and O^T += V^T P^T of this step, issued interleaved so that
// consecutive products never share an accumulator (the S^T products form
// only 2G dependent chains of D/32 links each).
struct NoHook {
    __device__ __forceinline__ void operator()(int) const {}
};

template <int D, int G, typename Hook = NoHook>
__device__ __forceinline__ void qk_pv(const bf16x8 (&ka)[D / 32][2], const bf16x8 (&qf)[G][D / 32],
                                      const f32x4 (&s0)[G], f32x4 (&sn)[2][G],
                                      const bf16x8 (&va)[D / 16], const bf16x2 (&pk)[G][4],
                                      f32x4 (&o)[G][D / 16], const Hook& hook = Hook()) {
    using GG = Geo<D>;
    constexpr int DPK = GG::DB / GG::KS;                // P.V column blocks per k-step
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int g = 0; g < G; ++g) sn[b][g] = s0[g];
#pragma unroll
    for (int ks = 0; ks < GG::KS; ++ks) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int g = 0; g < G; ++g)
                sn[b][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks][b], qf[g][ks], sn[b][g], 0, 0, 0);
#pragma unroll
        for (int db = ks * DPK; db < (ks + 1) * DPK; ++db)
#pragma unroll
            for (int g = 0; g < G; ++g)
                o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pack_p<G>(pk, g), o[g][db], 0, 0, 0);
        hook(ks);                                       // work issued between k-steps
    }
}

// O^T += V^T P^T for one 32-key step (the last step: no next scores).
template <int D, int G>
__device__ __forceinline__ void pv(const bf16x8 (&va)[D / 16], const bf16x2 (&pk)[G][4],
                                   f32x4 (&o)[G][D / 16]) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
        for (int g = 0; g < G; ++g)
            o[g][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pack_p<G>(pk, g), o[g][db], 0, 0, 0);
}

// O^T += V^T P^T for the lone 16-key granule at koff (K = 16 products).
template <int D, int G>
__device__ __forceinline__ void pv_half(const unsigned char* Vs, int koff, const bf16x2 (&pk)[G][2],
                                        f32x4 (&o)[G][D / 16], const LaneAddr& la) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
        const i16x4 va = __builtin_bit_cast(i16x4, v_operand<D>(Vs, koff, 0, db, la));
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bf16x4 b = {pk[g][0][0], pk[g][0][1], pk[g][1][0], pk[g][1][1]};
            o[g][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, __builtin_bit_cast(i16x4, b),
                                                                 o[g][db], 0, 0, 0);
        }
    }
}

// lgkmcnt(0) with no wait on the other counters (gfx9 encoding).
#define FSA_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4))

// The vector phase of a step runs at issue priority 1: 4-5% faster than none
// (720p, 1080p, stress; same-process A/B), so that a wave's softmax and operand
// reads go ahead of its SIMD partner's products and the partner's matrix phase
// follows without a gap.
__device__ __forceinline__ void prio_vector_begin() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_vector_end() { __builtin_amdgcn_s_setprio(0); }

// The slice walk of one workgroup. Each 32-key step t runs in two phases: a
// vector phase (the softmax of S_t, while this step's V operands and the next
// step's K operands load from LDS) and a matrix phase (S_{t+1} and P_t V_t,
// interleaved). Two waves share each SIMD (two workgroups per CU); one wave's
// vector phase overlaps the other's matrix phase, which the hardware does far
// better than mixing the two kinds of work within one wave.
// Chunks of kBK keys stream into a two-stage LDS ring by direct-to-LDS
// copies issued one chunk ahead. At the last step of a chunk the wave holds
// that step's V operands in registers, waits for the next chunk's copies and
// passes one barrier: no wave reads the old stage after it, so the copy of
// the chunk after next goes there. Every chunk but the last is full; the
// last holds 16 to kBK keys, whole 16-key granules. Scores are always
// computed for 32 keys: past the slice end a stage holds copies of the
// slice's last key (finite values) whose scores are never used.
template <int D, int G, int R>
__device__ __forceinline__ void attend(unsigned char* smem, const Slice& sl, const __bf16* Kh,
                                       const __bf16* Vh, const bf16x8 (&qf)[G][D / 32],
                                       const f32x4 (&s0)[G], const float (&shift)[G],
                                       float c, f32x4 (&o)[G][D / 16],
                                       float (&rs)[G], float (&m)[G], int wave, int lane) {
    using GG = Geo<D>;
    constexpr int SPC = kBK / 32;                       // 32-key steps per chunk
    const LaneAddr la = lane_addr(lane & 15, lane >> 4);
    const int nchunks = (sl.total + kBK - 1) / kBK;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;

    const unsigned smem_lds = unsigned(uintptr_t((lds_void*)smem));
    issue_chunk4<D>(smem_lds, sl, Kh, Vh, 0, wave, lane);
    FSA_WAIT_VMCNT(0);                                  // chunk 0 has landed
    __builtin_amdgcn_s_barrier();
    if (nchunks > 1) issue_chunk4<D>(smem_lds + GG::STAGE, sl, Kh, Vh, 1, wave, lane);

    f32x4 sv[2][G];
    scores<D, G, 2>(smem, 0, qf, s0, sv, la);
    int st = 0;                                         // stage of chunk ch
    for (int ch = 0; ch + 1 < nchunks; ++ch) {
        const unsigned char* S0 = smem + st * GG::STAGE;
#pragma unroll
        for (int s = 0; s < SPC; ++s) {
            bf16x8 va[GG::DB];
            load_v<D>(S0 + GG::TILE, 32 * s, va, la);
            bf16x8 ka[GG::KS][2];
            if (s + 1 < SPC) {
                load_k<D>(S0, 32 * (s + 1), ka, la);
            } else {
                FSA_WAIT_VMCNT(0);                      // chunk ch+1 has landed
                FSA_WAIT_LGKM0();                       // this step's V is in registers
                __builtin_amdgcn_s_barrier();
                if (R != kOnline && ch + 2 < nchunks)
                    issue_chunk4<D>(smem_lds + st * GG::STAGE, sl, Kh, Vh, ch + 2, wave, lane);
                st ^= 1;
                load_k<D>(smem + st * GG::STAGE, 0, ka, la);
            }
            bf16x2 pk[G][4];
            prio_vector_begin();
            softmax<D, G, R, 2>(sv, c, shift, m, rs, o, pk);
            prio_vector_end();
            __builtin_amdgcn_sched_barrier(0);
            if (R == kOnline && s + 1 == SPC) {
                // Online route: the copies of the chunk after next are issued
                // between the k-steps of the matrix phase, which measured faster
                // for it than issuing them right after the barrier (the fixed
                // route is faster the other way). Past the last chunk they
                // repeat the slice's last key into the free stage, never read.
                const unsigned dst = smem_lds + (st ^ 1) * GG::STAGE;
                constexpr int NI = GG::BLOCKS / 4;
                static_assert(NI <= GG::KS, "one copy group per k-step");
                qk_pv<D, G>(ka, qf, s0, sv, va, pk, o, [&](int ks) {
                    if (ks < NI) issue_group<D, 4>(dst, sl, Kh, Vh, ch + 2, wave, lane, ks);
                });
            } else {
                qk_pv<D, G>(ka, qf, s0, sv, va, pk, o);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The last chunk; sv holds the scores of its first step.
    const unsigned char* S0 = smem + st * GG::STAGE;
    const int left = sl.total - (nchunks - 1) * kBK;    // 16 .. kBK keys
    int k0 = 0;
    for (; k0 + 32 <= left; k0 += 32) {
        bf16x8 va[GG::DB];
        load_v<D>(S0 + GG::TILE, k0, va, la);
        bf16x2 pk[G][4];
        if (k0 + 32 < left) {
            bf16x8 ka[GG::KS][2];
            load_k<D>(S0, k0 + 32, ka, la);
            softmax<D, G, R, 2>(sv, c, shift, m, rs, o, pk);
            qk_pv<D, G>(ka, qf, s0, sv, va, pk, o);
        } else {
            softmax<D, G, R, 2>(sv, c, shift, m, rs, o, pk);
            pv<D, G>(va, pk, o);
        }
    }
    if (left & 16) {                                    // the lone granule at k0
        bf16x2 pk[G][2];
        softmax<D, G, R, 1>(sv, c, shift, m, rs, o, pk);
        pv_half<D, G>(S0 + GG::TILE, k0, pk, o, la);
    }
    FSA_WAIT_VMCNT(0);                                  // no copy may outlive the workgroup
}

// A wave that owns no query rows (past the last unit of its frame) still
// moves its share of every chunk and passes the same barriers as the waves
// that compute, in the same order, but issues no matrix or softmax work. Its
// share follows the route of the workgroup: in the loop, the fixed route
// issues whole chunks from the copy waves and the online route has every wave
// issue its own groups.
template <int D>
__device__ __forceinline__ void copy_only(unsigned char* smem, const Slice& sl, const __bf16* Kh,
                                          const __bf16* Vh, bool fixed, int wave, int lane) {
    using GG = Geo<D>;
    const int nchunks = (sl.total + kBK - 1) / kBK;
    const unsigned smem_lds = unsigned(uintptr_t((lds_void*)smem));
    issue_chunk4<D>(smem_lds, sl, Kh, Vh, 0, wave, lane);
    FSA_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (nchunks > 1) issue_chunk4<D>(smem_lds + GG::STAGE, sl, Kh, Vh, 1, wave, lane);
    int st = 0;
    for (int ch = 0; ch + 1 < nchunks; ++ch) {
        FSA_WAIT_VMCNT(0);
        __builtin_amdgcn_s_barrier();
        if (ch + 2 < nchunks) {
            if (fixed) {
                issue_chunk4<D>(smem_lds + st * GG::STAGE, sl, Kh, Vh, ch + 2, wave, lane);
            } else {
#pragma unroll
                for (int i = 0; i < GG::BLOCKS / 4; ++i)
                    issue_group<D, 4>(smem_lds + st * GG::STAGE, sl, Kh, Vh, ch + 2, wave, lane, i);
            }
        }
        st ^= 1;
    }
    FSA_WAIT_VMCNT(0);
}

// An empty asm statement that may touch any memory: LDS reads are neither
// hoisted above nor sunk below it (a barrier alone does not order them).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// The slice walk of an 8-wave workgroup (256 rows, one workgroup per CU, so
// the two waves of each SIMD belong to the same workgroup). Chunks of kBK
// keys stream into a 4-stage LDS ring; every wave copies its own blocks of
// every chunk, and the waves meet at one barrier per pair of chunks. A
// microbenchmark of this step's instruction mix measured that well ahead of a
// barrier per chunk: each barrier lines up the two waves of a SIMD, and only
// between barriers do their vector and matrix phases drift apart and overlap.
// Chunk c lives in stage c % 4. Before the walk, chunks 0-3 are issued, 0 and
// 1 have landed, and the waves pass one barrier. Barrier p sits in step
// 4p + 3 (the last step of chunks 2p and 2p + 1), between that step's V reads
// and the next step's K reads. Before it each wave waits for its own copies
// (chunks 2p + 2 and 2p + 3, issued at barrier p - 1) and for its own reads,
// so after it chunks 2p + 2 and 2p + 3 are visible to every wave and no wave
// reads the stages of chunks 2p and 2p + 1 again: the copies of chunks 2p + 4
// and 2p + 5 go there at once. The steps themselves are those of attend.
template <int D>
__device__ __forceinline__ void walk8_prologue(unsigned lds0, const Slice& sl, const __bf16* Kh,
                                               const __bf16* Vh, int nchunks, int wave, int lane) {
    using GG = Geo<D>;
    constexpr int CPW = 2 * (GG::BLOCKS / 4);          // copies per copying wave per chunk
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
        if (ch < nchunks) issue_chunk8<D>(lds0 + ch * GG::STAGE, sl, Kh, Vh, ch, wave, lane);
    // chunks 0 and 1 have landed; 2 and 3 may still be in flight (waves 4-7
    // have issued nothing, so every wait passes at once for them)
    if (nchunks >= 4) FSA_WAIT_VMCNT(2 * CPW);
    else if (nchunks == 3) FSA_WAIT_VMCNT(CPW);
    else FSA_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

template <int D>
__device__ __forceinline__ void walk8_barrier(unsigned lds0, const Slice& sl, const __bf16* Kh,
                                              const __bf16* Vh, int pair, int nchunks, int wave,
                                              int lane) {
    using GG = Geo<D>;
    compiler_fence();
    FSA_WAIT_VMCNT(0);                                  // my copies of chunks 2p+2, 2p+3
    FSA_WAIT_LGKM0();                                   // my reads of chunks 2p, 2p+1
    __builtin_amdgcn_s_barrier();
    compiler_fence();
#pragma unroll
    for (int ch = 2 * pair + 4; ch < 2 * pair + 6; ++ch)
        if (ch < nchunks) issue_chunk8<D>(lds0 + (ch & 3) * GG::STAGE, sl, Kh, Vh, ch, wave, lane);
}

template <int D, int G, int R>
__device__ __forceinline__ void attend8(unsigned char* smem, const Slice& sl, const __bf16* Kh,
                                        const __bf16* Vh, const bf16x8 (&qf)[G][D / 32],
                                        const f32x4 (&s0)[G], const float (&shift)[G],
                                        float c, f32x4 (&o)[G][D / 16],
                                        float (&rs)[G], float (&m)[G], int wave, int lane) {
    using GG = Geo<D>;
    const LaneAddr la = lane_addr(lane & 15, lane >> 4);
    const int nchunks = (sl.total + kBK - 1) / kBK;
    const int nsteps = (sl.total + 31) >> 5;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;
    const unsigned lds0 = unsigned(uintptr_t((lds_void*)smem));
    walk8_prologue<D>(lds0, sl, Kh, Vh, nchunks, wave, lane);

    f32x4 sv[2][G];
    scores<D, G, 2>(smem, 0, qf, s0, sv, la);
    for (int t = 0; t + 1 < nsteps; ++t) {
        const unsigned char* S0 = smem + ((t >> 1) & 3) * GG::STAGE;
        bf16x8 va[GG::DB];
        load_v<D>(S0 + GG::TILE, 32 * (t & 1), va, la);
        if ((t & 3) == 3) walk8_barrier<D>(lds0, sl, Kh, Vh, t >> 2, nchunks, wave, lane);
        const int t1 = t + 1;
        bf16x8 ka[GG::KS][2];
        load_k<D>(smem + ((t1 >> 1) & 3) * GG::STAGE, 32 * (t1 & 1), ka, la);
        bf16x2 pk[G][4];
        prio_vector_begin();
        softmax<D, G, R, 2>(sv, c, shift, m, rs, o, pk);
        prio_vector_end();
        __builtin_amdgcn_sched_barrier(0);
        qk_pv<D, G>(ka, qf, s0, sv, va, pk, o);
        __builtin_amdgcn_sched_barrier(0);
    }
    // The last step: 32 keys, or the slice's lone last 16-key granule.
    const int t = nsteps - 1;
    const unsigned char* S0 = smem + ((t >> 1) & 3) * GG::STAGE;
    if (sl.total - 32 * t >= 32) {
        bf16x8 va[GG::DB];
        load_v<D>(S0 + GG::TILE, 32 * (t & 1), va, la);
        bf16x2 pk[G][4];
        softmax<D, G, R, 2>(sv, c, shift, m, rs, o, pk);
        pv<D, G>(va, pk, o);
    } else {
        bf16x2 pk[G][2];
        softmax<D, G, R, 1>(sv, c, shift, m, rs, o, pk);
        pv_half<D, G>(S0 + GG::TILE, 32 * (t & 1), pk, o, la);
    }
    FSA_WAIT_VMCNT(0);                                  // no copy may outlive the workgroup
}

// A wave of an 8-wave workgroup that owns no query rows: the same copies and
// barriers as attend8, in the same order, with no matrix or softmax work.
template <int D>
__device__ __forceinline__ void copy_only8(unsigned char* smem, const Slice& sl, const __bf16* Kh,
                                           const __bf16* Vh, int wave, int lane) {
    const int nchunks = (sl.total + kBK - 1) / kBK;
    const int nsteps = (sl.total + 31) >> 5;
    const unsigned lds0 = unsigned(uintptr_t((lds_void*)smem));
    walk8_prologue<D>(lds0, sl, Kh, Vh, nchunks, wave, lane);
    for (int t = 3; t + 1 < nsteps; t += 4) walk8_barrier<D>(lds0, sl, Kh, Vh, t >> 2, nchunks, wave, lane);
    FSA_WAIT_VMCNT(0);
}

// The slice walk of a workgroup whose frame has a single row unit left for it
// (T = 3600 leaves one 16-row granule after 28 full workgroups): rather than
// one wave computing while the others only stage keys, every wave takes the
// same unit, and wave w computes on the w-th 16-key granule of every chunk,
// all waves staging and passing the barriers as usual. Each wave ends with
// partial sums over its granules (and, on the online route, its running
// max), which combine_split adds up.
template <int D, int G, int R>
__device__ __forceinline__ void attend_split(unsigned char* smem, const Slice& sl,
                                             const __bf16* Kh, const __bf16* Vh,
                                             const bf16x8 (&qf)[G][D / 32], const f32x4 (&s0)[G],
                                             const float (&shift)[G], float c,
                                             f32x4 (&o)[G][D / 16], float (&rs)[G],
                                             float (&m)[G], int wave, int lane) {
    using GG = Geo<D>;
    const LaneAddr la = lane_addr(lane & 15, lane >> 4);
    const int nchunks = (sl.total + kBK - 1) / kBK;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;
    const unsigned smem_lds = unsigned(uintptr_t((lds_void*)smem));
    issue_chunk4<D>(smem_lds, sl, Kh, Vh, 0, wave, lane);
    FSA_WAIT_VMCNT(0);
    __builtin_amdgcn_s_barrier();
    if (nchunks > 1) issue_chunk4<D>(smem_lds + GG::STAGE, sl, Kh, Vh, 1, wave, lane);
    int st = 0;
    for (int ch = 0; ch < nchunks; ++ch) {
        if (ch * kBK + 16 * wave < sl.total) {                  // this wave's granule exists
            const unsigned char* S0 = smem + st * GG::STAGE;
            f32x4 sv[2][G];
#pragma unroll
            for (int g = 0; g < G; ++g) sv[1][g] = f32x4{0.f, 0.f, 0.f, 0.f};
            scores<D, G, 1>(S0, 16 * wave, qf, s0, sv, la);
            bf16x2 pk[G][2];
            softmax<D, G, R, 1>(sv, c, shift, m, rs, o, pk);
            pv_half<D, G>(S0 + GG::TILE, 16 * wave, pk, o, la);
        }
        if (ch + 1 < nchunks) {
            FSA_WAIT_VMCNT(0);                                  // chunk ch+1 has landed
            FSA_WAIT_LGKM0();                                   // no read of the old stage is pending
            __builtin_amdgcn_s_barrier();
            if (ch + 2 < nchunks)
                issue_chunk4<D>(smem_lds + st * GG::STAGE, sl, Kh, Vh, ch + 2, wave, lane);
            st ^= 1;
        }
    }
    FSA_WAIT_VMCNT(0);
}

// The 8-wave counterpart of attend_split: a workgroup left with a single row
// unit (T = 3600 leaves one 16-row granule after 14 full 256-row workgroups).
// Every wave takes that unit; wave w computes on the w-th 16-key granule of
// every pair of chunks (chunk 2p + w / 4, granule w % 4), all waves passing
// the barriers of the ring as in attend8. combine_split adds the partials up.
template <int D, int G, int R>
__device__ __forceinline__ void attend_split8(unsigned char* smem, const Slice& sl,
                                              const __bf16* Kh, const __bf16* Vh,
                                              const bf16x8 (&qf)[G][D / 32], const f32x4 (&s0)[G],
                                              const float (&shift)[G], float c,
                                              f32x4 (&o)[G][D / 16], float (&rs)[G],
                                              float (&m)[G], int wave, int lane) {
    using GG = Geo<D>;
    const LaneAddr la = lane_addr(lane & 15, lane >> 4);
    const int nchunks = (sl.total + kBK - 1) / kBK;
    const int nsteps = (sl.total + 31) >> 5;
    const int npairs = (nchunks + 1) >> 1;
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = -INFINITY;
    const unsigned lds0 = unsigned(uintptr_t((lds_void*)smem));
    walk8_prologue<D>(lds0, sl, Kh, Vh, nchunks, wave, lane);
    for (int p = 0; p < npairs; ++p) {
        const int ch = 2 * p + (wave >> 2), k0 = 16 * (wave & 3);
        if (ch * kBK + k0 < sl.total) {                         // this wave's granule exists
            const unsigned char* S0 = smem + (ch & 3) * GG::STAGE;
            f32x4 sv[2][G];
#pragma unroll
            for (int g = 0; g < G; ++g) sv[1][g] = f32x4{0.f, 0.f, 0.f, 0.f};
            scores<D, G, 1>(S0, k0, qf, s0, sv, la);
            bf16x2 pk[G][2];
            softmax<D, G, R, 1>(sv, c, shift, m, rs, o, pk);
            pv_half<D, G>(S0 + GG::TILE, k0, pk, o, la);
        }
        // the barrier of pair p sits in step 4p + 3, as in attend8
        if (4 * p + 3 + 1 < nsteps) walk8_barrier<D>(lds0, sl, Kh, Vh, p, nchunks, wave, lane);
    }
    FSA_WAIT_VMCNT(0);
}

// Floats per lane that a wave of a split workgroup hands over: its partial
// output accumulators, row sums and running maxima.
template <int D, int G>
constexpr int split_floats() { return G * (D / 16) * 4 + 2 * G; }

// Adds the partial results of a split workgroup's W waves into wave 0, in
// wave order (so the sum is deterministic), through the LDS the key ring used.
// The fixed route's partial sums share one shift and simply add; the online
// route rescales each to the largest running max first. Returns true in wave
// 0 only, which then holds the whole row sums and accumulators.
template <int D, int G, int W>
__device__ __forceinline__ bool combine_split(unsigned char* smem, f32x4 (&o)[G][D / 16],
                                              float (&rs)[G], float (&m)[G], float c, bool fixed,
                                              int wave, int lane) {
    constexpr int NF = split_floats<D, G>();
    float* buf = reinterpret_cast<float*>(smem);
    FSA_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();                               // the key ring is no longer read
    if (wave > 0) {
        float* mine = buf + (wave - 1) * NF * 64 + lane;
        int i = 0;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int db = 0; db < D / 16; ++db)
#pragma unroll
                for (int e = 0; e < 4; ++e) mine[64 * i++] = o[g][db][e];
#pragma unroll
        for (int g = 0; g < G; ++g) mine[64 * i++] = rs[g];
#pragma unroll
        for (int g = 0; g < G; ++g) mine[64 * i++] = m[g];
    }
    // s_barrier does not wait for a wave's LDS writes on gfx950 (and the
    // compiler adds no wait before a bare barrier): wait for them, or wave 0
    // may read partials that have not landed.
    FSA_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    if (wave > 0) return false;
    for (int w = 1; w < W; ++w) {
        const float* theirs = buf + (w - 1) * NF * 64 + lane;
        constexpr int RS = G * (D / 16) * 4, MX = RS + G;
        if (fixed) {
            int i = 0;
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int db = 0; db < D / 16; ++db)
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[g][db][e] += theirs[64 * i++];
#pragma unroll
            for (int g = 0; g < G; ++g) rs[g] += theirs[64 * (RS + g)];
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float mw = theirs[64 * (MX + g)];
                const float mx = fmaxf(m[g], mw);               // wave 0's max is finite
                const float a = __builtin_amdgcn_exp2f((m[g] - mx) * c);
                const float b = __builtin_amdgcn_exp2f((mw - mx) * c);   // 0 for a wave with no chunk
                m[g] = mx;
                rs[g] = rs[g] * a + theirs[64 * (RS + g)] * b;
#pragma unroll
                for (int db = 0; db < D / 16; ++db)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[g][db][e] = o[g][db][e] * a + theirs[64 * ((g * (D / 16) + db) * 4 + e)] * b;
            }
        }
    }
    return true;
}

// The slice walk of route R for a workgroup of W waves (split: the walk of
// a workgroup left with a single row unit).
template <int D, int G, int W, int R>
__device__ __forceinline__ void walk(bool split, unsigned char* smem, const Slice& sl,
                                     const __bf16* Kh, const __bf16* Vh,
                                     const bf16x8 (&qf)[G][D / 32], const f32x4 (&s0)[G],
                                     const float (&shift)[G], float c, f32x4 (&o)[G][D / 16],
                                     float (&rs)[G], float (&m)[G], int wave, int lane) {
    if (split) {
        if (W == 8) attend_split8<D, G, R>(smem, sl, Kh, Vh, qf, s0, shift, c, o, rs, m, wave, lane);
        else attend_split<D, G, R>(smem, sl, Kh, Vh, qf, s0, shift, c, o, rs, m, wave, lane);
    } else if (W == 8) {
        attend8<D, G, R>(smem, sl, Kh, Vh, qf, s0, shift, c, o, rs, m, wave, lane);
    } else {
        attend<D, G, R>(smem, sl, Kh, Vh, qf, s0, shift, c, o, rs, m, wave, lane);
    }
}

// LDS of a workgroup: the key ring (4 stages for 8 waves, 2 for 4 waves); a
// split workgroup reuses it to combine its waves' partials.
template <int D, int G, int W>
constexpr int fwd_lds_bytes() {
    constexpr int ring = (W == 8 ? 4 : 2) * Geo<D>::STAGE;
    constexpr int partials = (W - 1) * split_floats<D, G>() * 64 * 4;
    return ring > partials ? ring : partials;
}

// W waves of 16*G rows each; two waves per SIMD (<= 256 registers per lane):
// two 4-wave workgroups or one 8-wave workgroup per CU.
template <int D, int G, int W, bool PMAX>
__global__ __launch_bounds__(64 * W, 2) void fwd_bf16(const FwdArgs p) {
    constexpr int RF = kFixed | (PMAX ? kPmax : 0);      // this kernel's fixed routes
    constexpr int RQ = kFixedScaled | (PMAX ? kPmax : 0);
    using GG = Geo<D>;
    static_assert(W == 4 || W == 8, "4 or 8 waves");
    static_assert(G * D <= 256, "a wave's accumulators and query fragments fit 256 registers");
    __shared__ __attribute__((aligned(16))) unsigned char smem[fwd_lds_bytes<D, G, W>()];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lj = lane >> 4;

    const int L = xcd_remap(blockIdx.x, p.nwg);
    const int gq = L % p.groups_per_frame;
    const int t1 = pair_at(p, L / p.groups_per_frame, routes_mixed(p));
    const int f = frame_at(p.tab, t1 % p.F);
    const int bh = t1 / p.F;
    const int T = p.T;
    const Slice sl = slice_of(p.tab, f, p.KT);

    const size_t base = size_t(bh) * p.N * D, kbase = size_t(bh) * p.NK * D;
    const __bf16* Qh = static_cast<const __bf16*>(p.Q) + base;
    bool fixed = use_fixed(p, bh, f);                    // uniform per workgroup
    const __bf16* Kh = static_cast<const __bf16*>(p.K) + kbase;
    const __bf16* Vh = static_cast<const __bf16*>(p.V) + kbase;
    __bf16* Oh = static_cast<__bf16*>(p.O) + base;

    // A wave owns granules unit*G .. unit*G+G-1 of frame f. Granules past the
    // frame (the tail of a frame whose granule count G does not divide)
    // repeat the frame's last granule and are not stored: every computing
    // wave runs the same loop, with no predicate inside it. A wave wholly
    // past the last unit only helps stage the keys, except in a workgroup
    // left with a single unit: there every wave takes that unit and a share
    // of the key chunks (attend_split, attend_split8).
    const int first_unit = gq * W;
    const bool split = p.units_per_frame - first_unit == 1;   // uniform
    const int unit = split ? first_unit : first_unit + wave;
    const int ngran = T >> 4;
    const int nvalid = max(0, min(G, ngran - unit * G));     // uniform per wave
    const int uwave = __builtin_amdgcn_readfirstlane(wave);
    const bool idle = __builtin_amdgcn_readfirstlane(nvalid) == 0;
    if (p.mode == FSA_MODE_AUTO_ROWS) {
        // The workgroup takes the fixed max iff every one of its rows has its
        // gap bound ||q_i|| R_S - q_i.dslice within the limit: each wave
        // reduces its rows, the waves meet once in LDS (idle waves too).
        __shared__ float wave_gap[W];
        float g = -INFINITY;
        if (!idle) {
            const float rsl = p.rslice[size_t(bh) * p.F + f];
            const float* dsl = p.dslice + (size_t(bh) * p.F + f) * D;
#pragma unroll
            for (int gg = 0; gg < G; ++gg) {
                const int row = f * T + 16 * min(unit * G + gg, ngran - 1) + ln;
                float dq = 0.f;
#pragma unroll
                for (int ks = 0; ks < GG::KS; ++ks) {
                    const bf16x8 q = *reinterpret_cast<const bf16x8*>(Qh + size_t(row) * D + 32 * ks + 8 * lj);
#pragma unroll
                    for (int e = 0; e < 8; ++e) dq = fmaf(float(q[e]), dsl[32 * ks + 8 * lj + e], dq);
                }
                dq += __shfl_xor(dq, 16, 64);
                dq += __shfl_xor(dq, 32, 64);
                g = fmaxf(g, p.qnorm[size_t(bh) * p.N + row] * rsl - dq);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) g = fmaxf(g, __shfl_xor(g, o, 64));
        }
        if (lane == 0) wave_gap[wave] = g;
        __syncthreads();
        float wg = wave_gap[0];
#pragma unroll
        for (int w = 1; w < W; ++w) wg = fmaxf(wg, wave_gap[w]);
        fixed = row_gap_ok(wg, p.c);
    }
    if (idle) {
        if (W == 8) copy_only8<D>(smem, sl, Kh, Vh, uwave, lane);
        else copy_only<D>(smem, sl, Kh, Vh, fixed, uwave, lane);
        return;
    }
    const float c = p.c;

    bf16x8 qf[G][GG::KS];
    float shift[G], rs[G];
    f32x4 o[G][GG::DB];
    const float rsl = p.rslice[size_t(bh) * p.F + f];
    bool wide = false;                                   // some row's bound above the limit
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int row = f * T + 16 * min(unit * G + g, ngran - 1) + ln;
#pragma unroll
        for (int ks = 0; ks < GG::KS; ++ks)
            qf[g][ks] = *reinterpret_cast<const bf16x8*>(Qh + size_t(row) * D + 32 * ks + 8 * lj);
        shift[g] = p.qnorm[size_t(bh) * p.N + row] * rsl;     // ||q_i|| R_S
        wide |= shift[g] * c > FSA_SCALED_LIMIT;
        rs[g] = 0.f;
#pragma unroll
        for (int db = 0; db < GG::DB; ++db) o[g][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // The scaled fixed route (taken by a wave whose rows all have c ||q_i|| R_S
    // within FSA_SCALED_LIMIT): the query fragments carry c, rounded to bf16
    // once here, q'_i = bf16(c q_i), and the products start from minus the
    // row's shift ||q'_i|| R_S + q'_i.mu, the Cauchy-Schwarz bound taken on
    // q'_i itself. The score products then yield the exponents of exp2 with no
    // vector operation per score, and no probability exceeds 1. The route
    // computes the fixed-max softmax of q'_i: the rounding moves each exponent
    // by at most 2^-9 c ||q_i|| ||k_j - mu|| <= 2^-4 beside a part common to
    // the row that cancels in the normalisation. Other fixed waves (rows with
    // keys spread wider) take the exact route: the shift
    // c (||q_i|| R_S + q_i.mu) on the query as given, applied per score.
    // The 4 lanes holding a row's columns add their partial sums in the same
    // pairing order, so all 4 get the same values.
    const float* muh = p.mu + size_t(bh) * D;
    const f32x4 zero[G] = {};
    float m[G];
    if (!fixed) {
        walk<D, G, W, kOnline>(split, smem, sl, Kh, Vh, qf, zero, shift, c, o, rs, m, uwave, lane);
    } else if (__builtin_amdgcn_ballot_w64(wide) == 0) {
        f32x4 s0[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float ss = 0.f, qm = 0.f;
#pragma unroll
            for (int ks = 0; ks < GG::KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const __bf16 x = __bf16(float(qf[g][ks][e]) * c);
                    qf[g][ks][e] = x;
                    ss = fmaf(float(x), float(x), ss);
                    qm = fmaf(float(x), muh[32 * ks + 8 * lj + e], qm);
                }
            ss += __shfl_xor(ss, 16, 64);
            ss += __shfl_xor(ss, 32, 64);
            qm += __shfl_xor(qm, 16, 64);
            qm += __shfl_xor(qm, 32, 64);
            const float z = -fmaf(sqrtf(ss), rsl, qm);
            s0[g] = f32x4{z, z, z, z};
        }
        walk<D, G, W, RQ>(split, smem, sl, Kh, Vh, qf, s0, shift, c, o, rs, m, uwave, lane);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float qm = 0.f;
#pragma unroll
            for (int ks = 0; ks < GG::KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    qm = fmaf(float(qf[g][ks][e]), muh[32 * ks + 8 * lj + e], qm);
            qm += __shfl_xor(qm, 16, 64);
            qm += __shfl_xor(qm, 32, 64);
            shift[g] = (shift[g] + qm) * c;
        }
        walk<D, G, W, RF>(split, smem, sl, Kh, Vh, qf, zero, shift, c, o, rs, m, uwave, lane);
    }
    if (PMAX && fixed) {
        // the largest probability this wave formed (every lane holds p >= 0,
        // so the float bits order like unsigned integers)
        float pm = m[0];
#pragma unroll
        for (int g = 1; g < G; ++g) pm = fmaxf(pm, m[g]);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) pm = fmaxf(pm, __shfl_xor(pm, off, 64));
        if (lane == 0 && pm > 0.f) atomicMax(p.pmax, __float_as_uint(pm));
    }
    // (the kernels that record the fixed route's largest probability, a check
    // run in tests, keep direct stores: staging would spill their registers)
    if (split || PMAX) {
        if (split && !combine_split<D, G, W>(smem, o, rs, m, c, fixed, uwave, lane)) return;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (g >= nvalid) break;
            float tot = rs[g] + __shfl_xor(rs[g], 16, 64);
            tot += __shfl_xor(tot, 32, 64);
            const float inv = 1.0f / tot;
            const int row = f * T + 16 * (unit * G + g) + ln;
#pragma unroll
            for (int db = 0; db < GG::DB; ++db) {
                bf16x4 out;
#pragma unroll
                for (int i = 0; i < 4; ++i) out[i] = __bf16(o[g][db][i] * inv);
                *reinterpret_cast<bf16x4*>(Oh + size_t(row) * D + 16 * db + 4 * lj) = out;
            }
        }
        return;
    }
    // The wave's 16G x D output tile goes through its own 2*16G*D bytes of the
    // key ring (free once every computing wave has passed the barrier below;
    // the waves that only stage keys have returned), then out as whole rows,
    // 16 bytes a lane: half the store instructions, whole cache lines. In row
    // r, 16-byte segment s sits at s ^ (r & 7) and its two 8-byte halves trade
    // places when r & 8, so that the 16 rows one write instruction touches
    // fill 128 distinct bytes of banks and each row read takes whole lines.
    constexpr int RB2 = D * 2;                           // bytes per row
    constexpr int SPR = RB2 / 16;                        // 16-byte segments per row
    static_assert(W * 16 * G * RB2 <= fwd_lds_bytes<D, G, W>(), "staging fits the ring");
    const unsigned stage_out = unsigned(uintptr_t((lds_void*)smem)) + uwave * (16 * G * RB2);
    FSA_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float tot = rs[g] + __shfl_xor(rs[g], 16, 64);
        tot += __shfl_xor(tot, 32, 64);
        const float inv = 1.0f / tot;
        const int r = 16 * g + ln;
#pragma unroll
        for (int db = 0; db < GG::DB; ++db) {
            bf16x4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = __bf16(o[g][db][i] * inv);
            const unsigned seg = unsigned(2 * db + (lj >> 1)) ^ unsigned(r & 7);
            const unsigned half = unsigned(lj & 1) ^ unsigned((r >> 3) & 1);
            *(lds_bf16x4*)(stage_out + r * RB2 + seg * 16 + half * 8) = out;
        }
    }
    constexpr int RPR = 64 / SPR;                        // rows per read
#pragma unroll
    for (int i = 0; i < 16 * G / RPR; ++i) {
        const int r = RPR * i + lane / SPR, sg = lane % SPR;
        bf16x8 v = *(const lds_bf16x8*)(stage_out + r * RB2 + ((sg ^ (r & 7)) * 16));
        if ((r >> 3) & 1) v = __builtin_shufflevector(v, v, 4, 5, 6, 7, 0, 1, 2, 3);
        if (r < 16 * nvalid)
            *reinterpret_cast<bf16x8*>(Oh + size_t(f * T + 16 * unit * G + r) * D + 8 * sg) = v;
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
    const Slice sl = slice_of(p.tab, f, p.KT);
    const size_t base = size_t(bh) * p.N * D, kbase = size_t(bh) * p.NK * D;
    bool fixed = use_fixed(p, bh, f);
    const float* Qh = static_cast<const float*>(p.Q) + base;
    const float* Kh = static_cast<const float*>(p.K) + kbase;
    const float* Vh = static_cast<const float*>(p.V) + kbase;
    float* Oh = static_cast<float*>(p.O) + base;
    const float c = p.c;

    float q[D], o[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        q[e] = Qh[size_t(i) * D + e];
        o[e] = 0.f;
    }
    float qm = 0.f;                 // the fixed route scores K as given: shift by q.mu too
#pragma unroll
    for (int e = 0; e < D; ++e) qm = fmaf(q[e], p.mu[size_t(bh) * D + e], qm);
    const float bnd = p.qnorm[size_t(bh) * p.N + i] * p.rslice[size_t(bh) * p.F + f];
    if (p.mode == FSA_MODE_AUTO_ROWS) {        // this row's own gap bound
        const float* dsl = p.dslice + (size_t(bh) * p.F + f) * D;
        float dq = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) dq = fmaf(q[e], dsl[e], dq);
        fixed = row_gap_ok(bnd - dq, c);
    }
    const float shift = c * (bnd + qm);
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

template <int D, int G, int W>
void launch_bf16(const FwdArgs& a, bool pmax, hipStream_t stream) {
    if (pmax)
        hipLaunchKernelGGL((fwd_bf16<D, G, W, true>), dim3(a.nwg), dim3(64 * W), 0, stream, a);
    else
        hipLaunchKernelGGL((fwd_bf16<D, G, W, false>), dim3(a.nwg), dim3(64 * W), 0, stream, a);
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
    a.mu = reinterpret_cast<const float*>(ws + p.ws.mu);
    a.K = K;
    a.V = V;
    a.O = O;
    a.qnorm = reinterpret_cast<const float*>(ws + p.ws.qnorm);
    a.rslice = reinterpret_cast<const float*>(ws + p.ws.rslice);
    a.elig = reinterpret_cast<const uint8_t*>(ws + p.ws.elig);
    a.eligf = reinterpret_cast<const uint8_t*>(ws + p.ws.eligf);
    a.dslice = reinterpret_cast<const float*>(ws + p.ws.dslice);
    a.pmax = reinterpret_cast<unsigned*>(const_cast<char*>(ws) + p.ws.pmax);
    const bool pmax = (mode & FSA_MODE_RECORD_PMAX) != 0;
    mode &= ~FSA_MODE_RECORD_PMAX;
    a.c = scale * kLog2e;
    a.N = s.F * s.T;
    a.NK = int32_t(p.key_tokens());
    a.KT = p.key_span;
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
        const int G = p.forward.granules, W = p.forward.waves;
        if (s.d == 128 && G == 2 && W == 8) {
            launch_bf16<128, 2, 8>(a, pmax, stream);
        } else if (s.d == 128 && G == 2 && W == 4) {
            launch_bf16<128, 2, 4>(a, pmax, stream);
        } else if (s.d == 64 && G == 2 && W == 8) {
            launch_bf16<64, 2, 8>(a, pmax, stream);
        } else if (s.d == 64 && G == 2 && W == 4) {
            launch_bf16<64, 2, 4>(a, pmax, stream);
        } else {
            set_error("fsa_forward: no kernel for d=%d with %d granules and %d waves", s.d, G, W);
            return FSA_ERR_UNSUPPORTED;
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
