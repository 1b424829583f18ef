// workspace.h -- layout of the caller-owned device workspace.
//
// Rows are padded to a multiple of 8 (one row per XCD lane of the dispatch
// mapping).  Everything is plain device memory and needs no initial value:
// barrier arrivals carry the call's 56-bit epoch, so the first arrival of a
// call resets whatever the word held (a previous call, or another layout's
// data); generations are only compared for change; the candidate count is
// reset by the workgroup that publishes the crossing bin.
#pragma once

#include <stdint.h>

namespace nucleus {

constexpr int kCap = 8192;       // candidates per row handed to the resolver
constexpr int kMaxChunks = 64;   // split-row path limit: V <= 64 * 8192

// Per-row control block: barrier state and the values published at each
// phase.  128 bytes.
struct RowCtl {
    uint64_t arrive;     // (call epoch << 8) | arrivals at the current barrier
    uint32_t gen;        // barrier generation (bumped by the last arriver)
    uint32_t cand_n;     // candidates appended this call
    uint32_t mode;       // row mode (model.h)
    float m;             // row max
    uint32_t pad0;
    uint32_t cbin;       // crossing bin (mode P) / last candidate bin (mode K)
    uint32_t cut_key;    // key of the smallest kept logit (published for the probability pass)
    uint32_t count;      // kept count
    uint64_t tc;         // mode P threshold inside the crossing bin
    double a_above;      // mode P: weight of the bins above the crossing bin
    double s_total;      // weight of all survivors
    double s_keep;       // weight of the kept set
    uint32_t token;      // sampled token (published for the probability pass)
    uint32_t pad[13];
};
static_assert(sizeof(RowCtl) == 128, "RowCtl layout");

// Per-workgroup partial of the race: best packed (score, ~index), kept
// count, smallest kept key.
struct RacePart {
    uint64_t best;
    uint32_t count;
    uint32_t minkey;
};

struct Work {
    RowCtl* ctl;          // [rows]
    uint4* slot_a;        // [rows * K]: max bits, error flag, 0, 0
    uint64_t* slot_h;     // [rows * K][kBins] bin weights
    uint32_t* slot_c;     // [rows * K][kBins] bin counts (top-k rows)
    RacePart* slot_r;     // [rows * K]
    uint2* cand;          // [rows][kCap]: key, index
    int K;                // workgroups per row
    uint64_t epoch;       // this call's tag (56 bits), distinct for every call
    int64_t give_up_row;  // -1; else the row whose waits give up at once (failure-path tests)
};

// Per-row state of the row path (row_kernel publishes the decided state and
// the row's model for race_kernel and probs_kernel; race_kernel merges the
// race partials of a row's chunks into it and the row's last chunk writes
// the outputs back for probs_kernel).  256 bytes.
struct RowPathState {
    uint32_t mode;       // row mode (model.h)
    float m;             // row max
    uint32_t pad1;
    uint32_t cbin;       // crossing bin (mode P) / last candidate bin (mode K)
    uint64_t tc;         // mode P threshold inside the crossing bin
    double a_above;      // mode P: weight of the bins above the crossing bin
    double s_total;      // weight of all survivors
    float keep_lo;       // surely kept iff x >= keep_lo
    float cand_lo;       // candidate iff cand_lo <= x < keep_lo
    uint64_t best;       // merged race: max of (score bits << 32 | ~index)
    uint32_t count;      // merged race: kept tokens seen
    uint32_t minkey;     // merged race: smallest kept key
    uint32_t cand_n;     // candidates appended
    uint32_t done;       // chunks finished
    uint32_t token;      // outputs, for probs_kernel
    uint32_t out_count;
    uint32_t cut_key;
    uint32_t pad0;
    double s_keep;
    uint32_t pad[8];
    uint64_t model[16];  // the row's RowModel (model.h), 128 bytes reserved
};
static_assert(sizeof(RowPathState) == 256, "RowPathState layout");

struct RowWork {
    RowPathState* st;     // [rows]
    uint2* cand;          // [rows][kCap]: key, index
    int N;                // race_kernel: 2048-token items per row; probs_kernel: 8192-token chunks per row
};

__host__ __device__ inline int64_t padded_rows(int64_t B) { return (B + 7) / 8 * 8; }

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Byte offsets of each region for a batch of B rows with K workgroups each.
struct WorkLayout {
    size_t ctl, slot_a, slot_h, slot_c, slot_r, cand, total;
};

// Row-path workspace: [rows] RowPathState, then [rows][kCap] candidates.
inline size_t row_work_bytes(int64_t B, size_t* cand_off)
{
    const size_t rows = (size_t)padded_rows(B);
    const size_t off = align256(rows * sizeof(RowPathState));
    if (cand_off) *cand_off = off;
    return align256(off + rows * (size_t)kCap * 8);
}

inline WorkLayout work_layout(int64_t B, int K, int bins)
{
    const size_t rows = (size_t)padded_rows(B);
    const size_t wgs = rows * (size_t)K;
    WorkLayout L;
    size_t off = 0;
    L.ctl = off; off = align256(off + rows * sizeof(RowCtl));
    L.slot_a = off; off = align256(off + wgs * 16);
    L.slot_h = off; off = align256(off + wgs * (size_t)bins * 8);
    L.slot_c = off; off = align256(off + wgs * (size_t)bins * 4);
    L.slot_r = off; off = align256(off + wgs * sizeof(RacePart));
    L.cand = off; off = align256(off + rows * (size_t)kCap * 8);
    L.total = off;
    return L;
}

}  // namespace nucleus
