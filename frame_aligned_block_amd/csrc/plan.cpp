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
// SIMD can hold in registers (output accumulators plus query fragments).
int32_t kernel_granules(int32_t d) { return d == 128 ? 2 : 4; }

int32_t pick_bk(int32_t T) {
    int32_t n = T / 16;
    for (int32_t g = 4; g >= 1; --g)
        if (n % g == 0) return 16 * g;
    return 16;
}

}  // namespace

extern "C" fsa_status fsa_plan_create(const fsa_shape* s_in, fsa_plan** out) {
    using namespace fsa;
    if (!s_in || !out) {
        set_error("fsa_plan_create: NULL argument");
        return FSA_ERR_INVALID_ARG;
    }
    *out = nullptr;
    fsa_shape s = *s_in;
    if (s.B < 1 || s.H < 1 || s.F < 1 || s.T < 1 || s.window < 0 ||
        s.ref_frame < 0 || s.ref_frame >= s.F || s.bq < 0 || s.bk < 0 ||
        (s.dtype != FSA_BF16 && s.dtype != FSA_F32)) {
        set_error("fsa_plan_create: invalid shape (B=%d H=%d F=%d T=%d window=%d ref=%d bq=%d bk=%d dtype=%d)",
                  s.B, s.H, s.F, s.T, s.window, s.ref_frame, s.bq, s.bk, s.dtype);
        return FSA_ERR_INVALID_ARG;
    }
    if (s.T % 16 != 0) {
        set_error("fsa_plan_create: T=%d is not a multiple of 16; frame-aligned blocks need 16 | T", s.T);
        return FSA_ERR_UNSUPPORTED;
    }
    if (s.d != 64 && s.d != 128) {
        set_error("fsa_plan_create: head width d=%d unsupported (64 or 128)", s.d);
        return FSA_ERR_UNSUPPORTED;
    }
    if (s.F > FSA_MAX_FRAMES) {
        set_error("fsa_plan_create: F=%d above the limit %d", s.F, FSA_MAX_FRAMES);
        return FSA_ERR_UNSUPPORTED;
    }
    const int64_t N = int64_t(s.F) * s.T;
    if (int64_t(s.B) * s.H * N * s.d > 0x7fffffffLL) {
        set_error("fsa_plan_create: B*H*N*d above 2^31-1 elements");
        return FSA_ERR_UNSUPPORTED;
    }
    for (int32_t b : {s.bq, s.bk}) {
        if (b != 0 && (b % 16 != 0 || s.T % b != 0)) {
            set_error("fsa_plan_create: block size %d is not a multiple of 16 dividing T=%d", b, s.T);
            return FSA_ERR_INVALID_ARG;
        }
    }

    fsa_plan* p = new (std::nothrow) fsa_plan();
    if (!p) {
        set_error("fsa_plan_create: out of host memory");
        return FSA_ERR_NOMEM;
    }
    try {
        if (s.bq == 0) s.bq = pick_bq(s.T);
        if (s.bk == 0) s.bk = pick_bk(s.T);
        p->shape = s;

        // ---- slices and the per-frame run table
        p->slice_size.assign(s.F, 0);
        std::vector<std::pair<int32_t, int32_t>> weight;   // (-|S|, f)
        for (int32_t f = 0; f < s.F; ++f) {
            int32_t lo = std::max(0, f - s.window), hi = std::min(s.F - 1, f + s.window);
            // runs in ascending frame order: the window, and the reference frame
            // when it lies outside the window (merged if adjacent).
            int32_t a0 = lo, l0 = hi - lo + 1, a1 = 0, l1 = 0;
            if (s.ref_frame < lo) {
                if (s.ref_frame == lo - 1) { a0 = s.ref_frame; l0 += 1; }
                else { a1 = a0; l1 = l0; a0 = s.ref_frame; l0 = 1; }
            } else if (s.ref_frame > hi) {
                if (s.ref_frame == hi + 1) { l0 += 1; }
                else { a1 = s.ref_frame; l1 = 1; }
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
        p->n_kblocks = int32_t(N / s.bk);
        p->row_ptr.reserve(p->n_qblocks + 1);
        p->row_ptr.push_back(0);
        p->qframe.reserve(p->n_qblocks);
        p->runs.reserve(size_t(p->n_qblocks) * 4);
        for (int32_t qb = 0; qb < p->n_qblocks; ++qb) {
            const int32_t f = int32_t(int64_t(qb) * s.bq / s.T);
            int32_t nrun = 0, r[4] = {0, 0, 0, 0};
            for (int32_t kb = 0; kb < p->n_kblocks; ++kb) {
                const int32_t g = int32_t(int64_t(kb) * s.bk / s.T);
                if (!in_slice(s.F, s.window, s.ref_frame, f, g)) continue;
                p->col_idx.push_back(kb);
                const int32_t a = kb * s.bk, e = a + s.bk;
                if (nrun > 0 && r[2 * (nrun - 1) + 1] == a) r[2 * (nrun - 1) + 1] = e;
                else {
                    if (nrun == 2) {   // cannot happen for window U {ref}
                        set_error("fsa_plan_create: internal error, more than two key runs");
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
            const int32_t T = s.T;
            const int32_t e0 = int32_t(t & 0xff) * T, e1 = e0 + int32_t((t >> 8) & 0xff) * T;
            const int32_t e2 = int32_t((t >> 16) & 0xff) * T, e3 = e2 + int32_t(t >> 24) * T;
            const bool ok = r[0] == e0 && r[1] == e1 &&
                            ((t >> 24) == 0 ? (r[2] == 0 && r[3] == 0) : (r[2] == e2 && r[3] == e3));
            if (!ok) {
                set_error("fsa_plan_create: internal error, run table disagrees with tile list");
                delete p;
                return FSA_ERR_INVALID_ARG;
            }
        }
        int64_t total = 0;
        for (int32_t f = 0; f < s.F; ++f) total += p->slice_size[f];
        p->valid_pairs = total * int64_t(s.T) * s.T;

        // ---- forward geometry: each wave takes `granules` consecutive 16-row
        // granules of one frame; a frame's last unit may hold fewer.
        const int32_t granules = kernel_granules(s.d);
        p->forward.granules = granules;
        p->forward.units_per_frame = (s.T / 16 + granules - 1) / granules;
        p->forward.groups_per_frame = (p->forward.units_per_frame + kWaves - 1) / kWaves;
        p->forward.workgroups = int64_t(s.B) * s.H * s.F * p->forward.groups_per_frame;

        // ---- bounds geometry: parts never straddle a frame
        const int32_t parts = (s.T + 255) / 256;
        p->bounds.rows_per_part = (s.T + parts - 1) / parts;
        p->bounds.parts_per_frame = (s.T + p->bounds.rows_per_part - 1) / p->bounds.rows_per_part;

        // ---- workspace layout
        const size_t BH = size_t(s.B) * s.H;
        size_t off = 0;
        fsa_ws_layout& w = p->ws;
        w.mu = off;      off = align_up(off + BH * s.d * 4);
        w.qnorm = off;   off = align_up(off + BH * N * 4);
        w.rframe = off;  off = align_up(off + BH * s.F * 4);
        w.rslice = off;  off = align_up(off + BH * s.F * 4);
        w.stat = off;    off = align_up(off + BH * 4);
        w.elig = off;    off = align_up(off + BH);
        w.statf = off;   off = align_up(off + BH * s.F * 4);
        w.eligf = off;   off = align_up(off + BH * s.F);
        const size_t nparts = size_t(s.F) * p->bounds.parts_per_frame;
        p->bounds.colsum = off;  off = align_up(off + BH * nparts * s.d * 4);
        p->bounds.partmax = off; off = align_up(off + BH * nparts * 4);
        p->bounds.partqmax = off; off = align_up(off + BH * nparts * 4);
        w.total = off;
    } catch (const std::bad_alloc&) {
        delete p;
        set_error("fsa_plan_create: out of host memory");
        return FSA_ERR_NOMEM;
    }
    *out = p;
    return FSA_OK;
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
