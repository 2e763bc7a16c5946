// planner.h - host-side constraint planner (no HIP dependency).
#pragma once
#include <stdint.h>

#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/dg.h"

namespace dg {

// Kernel families the planner can choose.
enum Family : int { F_TILED = 0, F_SKINNY_VALU = 1, F_SKINNY_MFMA = 2, F_SKINNY_E2M1 = 3 };

// One problem, after validation.
struct Problem {
    int64_t M, N, K;
    int path;        // Path
    int b_kmajor;    // 1: B stored N x K
    int out_type;    // Elt
    int epi;         // EpiKind
    int beta_nz;     // D is read
    int64_t k_pad = 0;   // pad_k: K elements past K (K is then the aligned part)
    int64_t ws_limit = -1;   // >= 0: prune plans whose partial sums need more bytes
                             // (a forced split is kept and checked by the caller)
};

struct Candidate {
    int family;
    int kernel_id;   // index within the family's catalogue
    int unit;        // dg_unit
    int mfma_m, mfma_n, mfma_k;
    int m_tile, n_tile, waves;
    int split_k, k_slice;
    int k_main, n_main, k_tail, n_tail;
    int lds, vgpr, agpr, waves_per_simd;
    int grid_x, grid_y;
    int64_t ws_bytes;
    double est_us, roof_us;
    std::string name;
    int k_pad = 0;   // pad_k: K elements added as one more partial slice by the tail kernel
};

struct PlanResult {
    dg_status status;
    std::string message;
    std::vector<Candidate> pareto;   // best first
    int enumerated = 0, pruned = 0;
    int ws_pruned = 0;   // candidates pruned by ws_limit
};

// Measurements of the tiled variants, from the probe's JSON description, by
// kernel name: the fraction of the probed MFMA rate a K step sustains, and the
// fixed time of one round of workgroups (prologue, epilogue and launch share),
// fitted from two K lengths of the same problem.
struct EffTable {
    std::unordered_map<std::string, double> eff, round_us;
    bool empty() const { return eff.empty(); }
    size_t size() const { return eff.size(); }
};

// Enumerate, prune, score, Pareto-filter.  Deterministic.  `eff` may be null
// (no calibration: the built-in fractions of the published peak are used).
PlanResult plan_problem(const Problem &pr, const dg_device_desc &desc, const dg_plan_opts &opts,
                        const EffTable *eff = nullptr);

// Fill the public description of a candidate.
void fill_info(const Candidate &c, dg_plan_info *out);

// Roofline time of the problem (microseconds) on the described device.
double roofline_us(const Problem &pr, const dg_device_desc &desc);

}  // namespace dg
