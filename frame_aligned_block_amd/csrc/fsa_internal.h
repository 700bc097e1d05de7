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
// runs[f] packs, in frame units, the up to two contiguous key ranges of frame
// f's slice, in ascending key order:
//   bits 0-7 start0, 8-15 len0, 16-23 start1, 24-31 len1   (len1 may be 0).
// order[] lists frames heaviest slice first (4 frame ids per word), which is
// the order workgroups are handed out in.
struct FrameTable {
    uint32_t runs[FSA_MAX_FRAMES + 1];
    uint32_t order[(FSA_MAX_FRAMES + 4) / 4];
};

// Query rows per wave = 16 * granules; a workgroup holds kWaves waves of
// consecutive row units of one frame.
#ifndef FSA_WAVES
#define FSA_WAVES 4
#endif
constexpr int kWaves = FSA_WAVES;
constexpr int kThreads = 64 * kWaves;

struct BoundsGeometry {
    int32_t rows_per_part;    // key/query rows one bounds workgroup reduces
    int32_t parts_per_frame;  // ceil(T / rows_per_part)
    size_t colsum;            // private ws offsets: float [BH][F*ppf][d]
    size_t partmax;           // float [BH][F*ppf]: max ||k_j - mu|| per part
    size_t partqmax;          // float [BH][F*ppf]: max ||q_i|| per part
};

struct ForwardGeometry {
    int32_t granules;          // 16-row granules per wave
    int32_t units_per_frame;   // ceil(T / (16 * granules)); the last may be partial
    int32_t groups_per_frame;  // ceil(units_per_frame / kWaves)
    int64_t workgroups;        // B * H * F * groups_per_frame
};

}  // namespace fsa

struct fsa_plan {
    fsa_shape shape;                 // bq, bk resolved
    int32_t n_qblocks = 0, n_kblocks = 0;
    std::vector<int32_t> row_ptr, col_idx, qframe, runs;   // runs: 4 per q-block
    std::vector<int32_t> slice_size;                       // |S(f)| per frame
    int64_t valid_pairs = 0;
    fsa::FrameTable table;
    fsa::BoundsGeometry bounds;
    fsa::ForwardGeometry forward;
    fsa_ws_layout ws;
};

namespace fsa {

// Thread-local last-error text (abi.cpp).
void set_error(const char* fmt, ...);

// Kernel launchers (bounds.hip, forward.hip). They assume a validated plan.
fsa_status launch_bounds(const fsa_plan& plan, const void* Q, const void* K, void* ws,
                         float scale, hipStream_t stream);
fsa_status launch_forward(const fsa_plan& plan, const void* Q, const void* K, const void* V,
                          void* O, const void* ws, float scale, int32_t mode, hipStream_t stream);

inline int32_t frame_order_at(const FrameTable& t, int32_t i) {
    return (t.order[i >> 2] >> (8 * (i & 3))) & 0xff;
}

}  // namespace fsa
