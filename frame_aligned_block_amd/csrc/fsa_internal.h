// Internal declarations shared by the host plan builder, the C-ABI layer and
// the HIP kernels of libfsa. Not part of the public interface (include/fsa.h).
#pragma once

#include <cstdint>
#include <cstddef>
#include <vector>

#include "../../include/fsa.h"

namespace fsa {

// Per-frame key runs as the kernels read them (kernel arguments, so they land
// in scalar registers / the constant cache: the gfx950 counterpart of feeding
// a small table to the kernel ahead of its grid, "Unchaining the Softmax" ¶2).
// runs[f] packs, in key-frame units, the up to two contiguous key ranges of
// query frame f's slice, in ascending key order:
//   bits 0-7 start0, 8-15 len0, 16-23 start1, 24-31 len1   (len1 may be 0).
// A key frame is T tokens of the chunk itself (self-attention) or the whole
// set of M reference tokens (cross-attention: every frame's slice is {0, 1}).
// order[] lists frames heaviest slice first (4 frame ids per word), which is
// the order workgroups are handed out in.
struct FrameTable {
    uint32_t runs[FSA_MAX_FRAMES + 1];
    uint32_t order[(FSA_MAX_FRAMES + 4) / 4];
};

// Rows of one side (queries or keys) cut into parts of at most 256 rows
// that never straddle a frame of that side.
struct Parts {
    int32_t span;             // rows per frame of this side
    int32_t frames;           // frames of this side
    int32_t rows_per_part;    // rows one bounds workgroup reduces
    int32_t per_frame;        // ceil(span / rows_per_part)
    int32_t count() const { return frames * per_frame; }
};

struct BoundsGeometry {
    Parts q;                  // query rows: F frames of T
    Parts k;                  // key rows: the key frames (F of T, or one of M)
    size_t colsum;            // private ws offsets: float [BH][k parts][d]
    size_t partmax;           // float [BH][k parts]: max ||k_j - mu|| per part
    size_t partqmax;          // float [BH][q parts]: max ||q_i|| per part
};

// The bf16 forward kernel's launch: workgroups of `waves` waves (4 or 8),
// each wave a unit of 16 * granules consecutive query rows of one frame, the
// waves of a workgroup consecutive units of the same frame.
struct ForwardGeometry {
    int32_t waves;             // waves per workgroup: 4 or 8
    int32_t granules;          // 16-row granules per wave
    int32_t units_per_frame;   // ceil(T / (16 * granules)); the last may be partial
    int32_t groups_per_frame;  // ceil(units_per_frame / waves)
    int64_t workgroups;        // B * H * F * groups_per_frame
};

// Fill the forward geometry of a plan for `waves` waves per workgroup.
void set_forward_geometry(fsa_plan& p, int32_t waves);

}  // namespace fsa

struct fsa_plan {
    fsa_shape shape;                 // bq, bk resolved
    // Key side. Self-attention: the chunk's own F frames of T tokens.
    // Cross-attention: one key frame of M reference tokens that every query
    // frame attends to. The run table counts in key frames of key_span tokens.
    bool cross = false;
    int32_t key_frames = 0, key_span = 0;
    int64_t key_tokens() const { return int64_t(key_frames) * key_span; }
    int32_t n_qblocks = 0, n_kblocks = 0;
    std::vector<int32_t> row_ptr, col_idx, qframe, runs;   // runs: 4 per q-block
    std::vector<int32_t> slice_size;                       // |S(f)| per frame
    int64_t valid_pairs = 0;
    fsa::FrameTable table;
    fsa::BoundsGeometry bounds;
    fsa::ForwardGeometry forward;
    fsa_ws_layout ws;
    size_t prep_ksum = 0;            // private ws: producer's key column sums, [BH][tiles][d]
    size_t prep_rscale = 0;          // private ws: producer's RMSNorm row scales, [B][N]
};

namespace fsa {

// The producer's RMSNorm epsilon and rotary base.
constexpr float kPrepEps = 1e-6f;
constexpr double kPrepBase = 10000.0;
// Tokens per producer tile (the key column sums are kept per tile).
constexpr int kPrepTile = 256;

// Thread-local last-error text (abi.cpp).
void set_error(const char* fmt, ...);

// Kernel launchers (bounds.hip, forward.hip). They assume a validated plan.
fsa_status launch_bounds(const fsa_plan& plan, const void* Q, const void* K, void* ws,
                         float scale, hipStream_t stream);
fsa_status launch_forward(const fsa_plan& plan, const void* Q, const void* K, const void* V,
                          void* O, const void* ws, float scale, int32_t mode, hipStream_t stream);
// Per-frame and per-slice radii, statistics and flags from the per-part maxima,
// and each slice's mean-key offset from the per-part key column sums (the
// workspace's colsum; both callers have written it).
fsa_status launch_bounds_finalize(const fsa_plan& plan, char* ws, float scale, hipStream_t stream);
// The producer (prep.hip).
fsa_status launch_prep_fold(const void* W, const float* gamma, void* Wp, int32_t C,
                            hipStream_t stream);
fsa_status launch_prep(const fsa_plan& plan, int32_t grid_w, const void* X, const void* Wp,
                       void* Q, void* K, void* V, void* ws, hipStream_t stream);
fsa_status launch_bounds_after_prep(const fsa_plan& plan, const void* K, void* ws, float scale,
                                    hipStream_t stream);

inline int32_t frame_order_at(const FrameTable& t, int32_t i) {
    return (t.order[i >> 2] >> (8 * (i & 3))) & 0xff;
}

}  // namespace fsa
