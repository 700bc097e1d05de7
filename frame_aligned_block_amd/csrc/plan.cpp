// Host builder of the frame-aligned tile plan (no HIP calls).
//
// Source: "HeyGen 与 Google Cloud：将 Avatar IV 部署到 TPU"
// (news.xcc.im/article/5328), "Deleting the Mask" ¶1-¶2: each frame attends to
// a window of nearby frames plus one global reference frame; with blocks that
// are multiples of 16 tokens dividing the frame span, every tile is entirely
// inside or outside the mask, so only live tiles are listed and none is
// partial, and the reference frame is just more full blocks in the same pass.
#include <algorithm>
#include <new>

#include "fsa_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool in_slice(int32_t F, int32_t window, int32_t ref, int32_t f, int32_t g) {
    (void)F;
    int32_t d = g > f ? g - f : f - g;
    return d <= window || g == ref;
}

// q-block size of the tile list when the caller leaves it open: the largest
// multiple of 16 up to 64 that divides T.
int32_t pick_bq(int32_t T) {
    const int32_t n = T / 16;
    for (int32_t g = 4; g >= 1; --g)
        if (n % g == 0) return 16 * g;
    return 16;
}

// 16-row granules per wave of the bf16 forward kernel: what two waves per
// SIMD can hold in registers (output accumulators plus query fragments) at
// d = 128; d = 64 keeps the same 32 rows per wave.
constexpr int32_t kGranules = 2;

// Waves per workgroup of the bf16 forward kernel ("Unchaining the Softmax" ¶3
// re-tunes block shapes together with the softmax). Two geometries exist:
//  * 4-wave workgroups (128 rows, two per CU): the two waves of a SIMD belong
//    to different workgroups and stay out of phase.
//  * 8-wave workgroups (256 rows, one per CU) stage each key chunk once for
//    twice the rows, so the CU moves half the bytes from L2 into LDS and
//    holds a higher clock under the chip's power limit; but their barriers
//    line up the two waves of every SIMD, which costs more cycles than the
//    clock gains.
// Same-process measurements of this kernel, 4 waves against 8: 3% faster at
// 720p, 1.0-1.6% at 1080p (T = 8160, where every 8-wave workgroup but a
// frame's last is full), 1% on stress, 4% on the cross workload, 15% on the
// small chunk, equal on the dense one. So every shape takes 4 waves, and
// fsa_plan_set_row_block selects 8.
int32_t pick_waves(const fsa_shape&) { return 4; }

// k-block size of the tile list when the caller leaves it open: as pick_bq,
// over the key frame's span.
int32_t pick_bk(int32_t T) {
    int32_t n = T / 16;
    for (int32_t g = 4; g >= 1; --g)
        if (n % g == 0) return 16 * g;
    return 16;
}

// Parts of at most 256 rows over `frames` frames of `span` rows each.
fsa::Parts make_parts(int32_t frames, int32_t span) {
    fsa::Parts g;
    g.span = span;
    g.frames = frames;
    const int32_t parts = (span + 255) / 256;
    g.rows_per_part = (span + parts - 1) / parts;
    g.per_frame = (span + g.rows_per_part - 1) / g.rows_per_part;
    return g;
}

// The builder behind fsa_plan_create (M = 0: self-attention over the chunk's
// own frames) and fsa_plan_create_cross (M reference tokens, one key frame).
fsa_status create_plan(const fsa_shape* s_in, int32_t M, fsa_plan** out, const char* who) {
    using namespace fsa;
    if (!s_in || !out) {
        set_error("%s: NULL argument", who);
        return FSA_ERR_INVALID_ARG;
    }
    *out = nullptr;
    const bool cross = M != 0;
    fsa_shape s = *s_in;
    if (s.B < 1 || s.H < 1 || s.F < 1 || s.T < 1 || s.window < 0 ||
        s.ref_frame < 0 || s.ref_frame >= s.F || s.bq < 0 || s.bk < 0 ||
        (s.dtype != FSA_BF16 && s.dtype != FSA_F32)) {
        set_error("%s: invalid shape (B=%d H=%d F=%d T=%d window=%d ref=%d bq=%d bk=%d dtype=%d)",
                  who, s.B, s.H, s.F, s.T, s.window, s.ref_frame, s.bq, s.bk, s.dtype);
        return FSA_ERR_INVALID_ARG;
    }
    if (cross && (M < 0 || s.window != 0 || s.ref_frame != 0)) {
        set_error("%s: M=%d must be positive and window=%d, ref_frame=%d both 0 (every query "
                  "attends to the whole reference set)", who, M, s.window, s.ref_frame);
        return FSA_ERR_INVALID_ARG;
    }
    if (s.T % 16 != 0) {
        set_error("%s: T=%d is not a multiple of 16; frame-aligned blocks need 16 | T", who, s.T);
        return FSA_ERR_UNSUPPORTED;
    }
    if (cross && M % 16 != 0) {
        set_error("%s: M=%d is not a multiple of 16; key blocks need 16 | M", who, M);
        return FSA_ERR_UNSUPPORTED;
    }
    if (s.d != 64 && s.d != 128) {
        set_error("%s: head width d=%d unsupported (64 or 128)", who, s.d);
        return FSA_ERR_UNSUPPORTED;
    }
    if (s.F > FSA_MAX_FRAMES) {
        set_error("%s: F=%d above the limit %d", who, s.F, FSA_MAX_FRAMES);
        return FSA_ERR_UNSUPPORTED;
    }
    const int64_t N = int64_t(s.F) * s.T;
    const int32_t KF = cross ? 1 : s.F, KT = cross ? M : s.T;
    const int64_t NK = int64_t(KF) * KT;
    if (int64_t(s.B) * s.H * N * s.d > 0x7fffffffLL ||
        int64_t(s.B) * s.H * NK * s.d > 0x7fffffffLL) {
        set_error("%s: B*H*N*d or B*H*(key tokens)*d above 2^31-1 elements", who);
        return FSA_ERR_UNSUPPORTED;
    }
    if (s.bq != 0 && (s.bq % 16 != 0 || s.T % s.bq != 0)) {
        set_error("%s: block size %d is not a multiple of 16 dividing T=%d", who, s.bq, s.T);
        return FSA_ERR_INVALID_ARG;
    }
    if (s.bk != 0 && (s.bk % 16 != 0 || KT % s.bk != 0)) {
        set_error("%s: block size %d is not a multiple of 16 dividing %s=%d", who, s.bk,
                  cross ? "M" : "T", KT);
        return FSA_ERR_INVALID_ARG;
    }

    fsa_plan* p = new (std::nothrow) fsa_plan();
    if (!p) {
        set_error("%s: out of host memory", who);
        return FSA_ERR_NOMEM;
    }
    try {
        if (s.bq == 0) s.bq = pick_bq(s.T);
        if (s.bk == 0) s.bk = pick_bk(KT);
        p->shape = s;
        p->cross = cross;
        p->key_frames = KF;
        p->key_span = KT;

        // ---- slices and the per-frame run table (in key frames)
        p->slice_size.assign(s.F, 0);
        std::vector<std::pair<int32_t, int32_t>> weight;   // (-|S|, f)
        for (int32_t f = 0; f < s.F; ++f) {
            int32_t a0 = 0, l0 = 1, a1 = 0, l1 = 0;
            if (!cross) {
                int32_t lo = std::max(0, f - s.window), hi = std::min(s.F - 1, f + s.window);
                // runs in ascending frame order: the window, and the reference
                // frame when it lies outside the window (merged if adjacent).
                a0 = lo; l0 = hi - lo + 1;
                if (s.ref_frame < lo) {
                    if (s.ref_frame == lo - 1) { a0 = s.ref_frame; l0 += 1; }
                    else { a1 = a0; l1 = l0; a0 = s.ref_frame; l0 = 1; }
                } else if (s.ref_frame > hi) {
                    if (s.ref_frame == hi + 1) { l0 += 1; }
                    else { a1 = s.ref_frame; l1 = 1; }
                }
            }
            p->table.runs[f] = uint32_t(a0) | uint32_t(l0) << 8 | uint32_t(a1) << 16 |
                               uint32_t(l1) << 24;
            p->slice_size[f] = l0 + l1;
            weight.push_back({-(l0 + l1), f});
        }
        std::stable_sort(weight.begin(), weight.end());
        std::fill(std::begin(p->table.order), std::end(p->table.order), 0u);
        for (int32_t i = 0; i < s.F; ++i)
            p->table.order[i >> 2] |= uint32_t(weight[i].second) << (8 * (i & 3));

        // ---- CSR tile list, built from the slice definition tile by tile
        p->n_qblocks = int32_t(N / s.bq);
        p->n_kblocks = int32_t(NK / s.bk);
        p->row_ptr.reserve(p->n_qblocks + 1);
        p->row_ptr.push_back(0);
        p->qframe.reserve(p->n_qblocks);
        p->runs.reserve(size_t(p->n_qblocks) * 4);
        for (int32_t qb = 0; qb < p->n_qblocks; ++qb) {
            const int32_t f = int32_t(int64_t(qb) * s.bq / s.T);
            int32_t nrun = 0, r[4] = {0, 0, 0, 0};
            for (int32_t kb = 0; kb < p->n_kblocks; ++kb) {
                const int32_t g = int32_t(int64_t(kb) * s.bk / KT);
                if (!cross && !in_slice(s.F, s.window, s.ref_frame, f, g)) continue;
                p->col_idx.push_back(kb);
                const int32_t a = kb * s.bk, e = a + s.bk;
                if (nrun > 0 && r[2 * (nrun - 1) + 1] == a) r[2 * (nrun - 1) + 1] = e;
                else {
                    if (nrun == 2) {   // cannot happen for window U {ref}
                        set_error("%s: internal error, more than two key runs", who);
                        delete p;
                        return FSA_ERR_INVALID_ARG;
                    }
                    r[2 * nrun] = a; r[2 * nrun + 1] = e; ++nrun;
                }
            }
            p->row_ptr.push_back(int32_t(p->col_idx.size()));
            p->qframe.push_back(f);
            for (int32_t i = 0; i < 4; ++i) p->runs.push_back(r[i]);
            // The kernels read the per-frame table; it must agree with the list.
            const uint32_t t = p->table.runs[f];
            const int32_t e0 = int32_t(t & 0xff) * KT, e1 = e0 + int32_t((t >> 8) & 0xff) * KT;
            const int32_t e2 = int32_t((t >> 16) & 0xff) * KT, e3 = e2 + int32_t(t >> 24) * KT;
            const bool ok = r[0] == e0 && r[1] == e1 &&
                            ((t >> 24) == 0 ? (r[2] == 0 && r[3] == 0) : (r[2] == e2 && r[3] == e3));
            if (!ok) {
                set_error("%s: internal error, run table disagrees with tile list", who);
                delete p;
                return FSA_ERR_INVALID_ARG;
            }
        }
        int64_t total = 0;
        for (int32_t f = 0; f < s.F; ++f) total += p->slice_size[f];
        p->valid_pairs = total * int64_t(s.T) * KT;

        // ---- forward geometry
        set_forward_geometry(*p, pick_waves(s));

        // ---- bounds geometry: parts never straddle a frame of their side
        p->bounds.q = make_parts(s.F, s.T);
        p->bounds.k = make_parts(KF, KT);

        // ---- workspace layout
        const size_t BH = size_t(s.B) * s.H;
        size_t off = 0;
        fsa_ws_layout& w = p->ws;
        w.mu = off;      off = align_up(off + BH * s.d * 4);
        w.qnorm = off;   off = align_up(off + BH * N * 4);
        w.rframe = off;  off = align_up(off + BH * KF * 4);
        w.rslice = off;  off = align_up(off + BH * s.F * 4);
        w.stat = off;    off = align_up(off + BH * 4);
        w.elig = off;    off = align_up(off + BH);
        w.statf = off;   off = align_up(off + BH * s.F * 4);
        w.eligf = off;   off = align_up(off + BH * s.F);
        w.dslice = off;  off = align_up(off + BH * s.F * s.d * 4);
        w.pmax = off;    off = align_up(off + 4);
        const size_t nkparts = size_t(p->bounds.k.count()), nqparts = size_t(p->bounds.q.count());
        p->bounds.colsum = off;  off = align_up(off + BH * nkparts * s.d * 4);
        p->bounds.partmax = off; off = align_up(off + BH * nkparts * 4);
        p->bounds.partqmax = off; off = align_up(off + BH * nqparts * 4);
        if (!cross) {        // the producer's per-tile key column sums
            const size_t tiles = size_t((N + kPrepTile - 1) / kPrepTile);
            p->prep_ksum = off; off = align_up(off + BH * tiles * s.d * 4);
            p->prep_rscale = off; off = align_up(off + size_t(s.B) * N * 4);
        }
        w.total = off;
    } catch (const std::bad_alloc&) {
        delete p;
        set_error("%s: out of host memory", who);
        return FSA_ERR_NOMEM;
    }
    *out = p;
    return FSA_OK;
}

}  // namespace

namespace fsa {

// Each wave takes `granules` consecutive 16-row granules of one frame; a
// frame's last unit may hold fewer, and its last workgroup fewer units.
void set_forward_geometry(fsa_plan& p, int32_t waves) {
    ForwardGeometry& g = p.forward;
    g.waves = waves;
    g.granules = kGranules;
    g.units_per_frame = (p.shape.T / 16 + kGranules - 1) / kGranules;
    g.groups_per_frame = (g.units_per_frame + waves - 1) / waves;
    g.workgroups = int64_t(p.shape.B) * p.shape.H * p.shape.F * g.groups_per_frame;
}

}  // namespace fsa

extern "C" fsa_status fsa_plan_create(const fsa_shape* shape, fsa_plan** out) {
    return create_plan(shape, 0, out, "fsa_plan_create");
}

extern "C" fsa_status fsa_plan_create_cross(const fsa_shape* shape, int32_t M, fsa_plan** out) {
    if (M <= 0) {
        fsa::set_error("fsa_plan_create_cross: M=%d must be positive", M);
        if (out) *out = nullptr;
        return FSA_ERR_INVALID_ARG;
    }
    return create_plan(shape, M, out, "fsa_plan_create_cross");
}

extern "C" void fsa_plan_destroy(fsa_plan* plan) { delete plan; }

extern "C" fsa_status fsa_plan_shape(const fsa_plan* plan, fsa_shape* out) {
    if (!plan || !out) {
        fsa::set_error("fsa_plan_shape: NULL argument");
        return FSA_ERR_INVALID_ARG;
    }
    *out = plan->shape;
    return FSA_OK;
}

extern "C" fsa_status fsa_plan_export(const fsa_plan* plan, int32_t* row_ptr, int32_t* col_idx,
                                      int32_t* qframe, int32_t* runs, int32_t* n_qblocks,
                                      int64_t* nnz) {
    if (!plan) {
        fsa::set_error("fsa_plan_export: NULL plan");
        return FSA_ERR_INVALID_ARG;
    }
    if (n_qblocks) *n_qblocks = plan->n_qblocks;
    if (nnz) *nnz = int64_t(plan->col_idx.size());
    if (row_ptr) std::copy(plan->row_ptr.begin(), plan->row_ptr.end(), row_ptr);
    if (col_idx) std::copy(plan->col_idx.begin(), plan->col_idx.end(), col_idx);
    if (qframe) std::copy(plan->qframe.begin(), plan->qframe.end(), qframe);
    if (runs) std::copy(plan->runs.begin(), plan->runs.end(), runs);
    return FSA_OK;
}

extern "C" int64_t fsa_plan_valid_pairs(const fsa_plan* plan) {
    return plan ? plan->valid_pairs : -1;
}

extern "C" int64_t fsa_plan_key_tokens(const fsa_plan* plan) {
    return plan ? plan->key_tokens() : -1;
}

extern "C" size_t fsa_workspace_bytes(const fsa_plan* plan) {
    return plan ? plan->ws.total : 0;
}

extern "C" fsa_status fsa_workspace_layout(const fsa_plan* plan, fsa_ws_layout* out) {
    if (!plan || !out) {
        fsa::set_error("fsa_workspace_layout: NULL argument");
        return FSA_ERR_INVALID_ARG;
    }
    *out = plan->ws;
    return FSA_OK;
}

extern "C" int32_t fsa_plan_row_block(const fsa_plan* plan) {
    if (!plan) return -1;
    if (plan->shape.dtype == FSA_F32) return 1;
    return 16 * plan->forward.granules * plan->forward.waves;
}

extern "C" fsa_status fsa_plan_set_row_block(fsa_plan* plan, int32_t rows) {
    if (!plan) {
        fsa::set_error("fsa_plan_set_row_block: NULL plan");
        return FSA_ERR_INVALID_ARG;
    }
    if (plan->shape.dtype == FSA_F32) {
        if (rows == 0 || rows == 1) return FSA_OK;
        fsa::set_error("fsa_plan_set_row_block: an fp32 plan computes one row per thread "
                       "(rows must be 0 or 1, got %d)", rows);
        return FSA_ERR_INVALID_ARG;
    }
    const int32_t per_wave = 16 * kGranules;
    int32_t waves;
    if (rows == 0) waves = pick_waves(plan->shape);
    else if (rows == 4 * per_wave) waves = 4;
    else if (rows == 8 * per_wave) waves = 8;
    else {
        fsa::set_error("fsa_plan_set_row_block: rows must be 0, %d or %d, got %d", 4 * per_wave,
                       8 * per_wave, rows);
        return FSA_ERR_INVALID_ARG;
    }
    fsa::set_forward_geometry(*plan, waves);
    return FSA_OK;
}
