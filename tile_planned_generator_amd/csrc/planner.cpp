// planner.cpp - the host-side constraint planner.
//
// The pages' tile planner models the GPU's physical limits as inequalities
// over the tile shape - shared memory used <= available, registers used <=
// the per-thread maximum, occupancy >= a target (70 % in their example) - and
// returns a Pareto-optimal set of (M_tile, N_tile, K_tile), with a K step that
// may change along K so that the last step still fills the matrix unit
// ([generator] DeepGEMM article, kwkr.cn, section 2.2, first layer; the
// planner run of section 3.2, step 2).  Their compiler enumerates tile shape x
// layout x granularity and prunes infeasible candidates before choosing
// ([overview] DeepGEMM article, section 4.1, stage 2).  The same procedure,
// re-derived for gfx950:
//   enumerate  the compiled kernel variants (tile shape and wave grid of the
//              tiled MFMA kernel; the skinny streaming kernels for small M)
//              x K split x K schedule;
//   prune      LDS bytes <= min(LDS per workgroup, the caller's limit);
//              VGPR+AGPR per lane <= 512 (AGPR <= 256);
//              waves per SIMD >= ceil(target occupancy x 8);
//              forced options; unit (MFMA or VALU) as requested;
//   score      a roofline-style model: per workgroup, max(MFMA time, LDS
//              time, L2 time) per K step, times the rounds of workgroups the
//              chip runs, against the HBM floor, plus store, reduce and
//              launch costs (the pages publish no cost model; this one is
//              the builder's);
//   choose     the Pareto set over (estimated time, LDS bytes, registers);
//              the minimum estimate wins, ties by fewer LDS bytes, then by
//              tile shape.  Deterministic.
#include "planner.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "catalogue.h"
#include "dg_args.h"

namespace dg {

namespace {

constexpr int SKINNY_A_LDS = 32768;   // must match skinny.hip
constexpr int E2M1_A_LDS = 32768;     // must match skinny.hip

const TiledShape k_tiled_shapes[] = {
#define DG_TS(path, kmaj, bm, bn, wm, wn, kr, ms) {path, kmaj, bm, bn, wm, wn, kr, ms},
    DG_TILED_CATALOGUE(DG_TS)
#undef DG_TS
};

struct ValuShape {
    int path, mr, lpr;
};
const ValuShape k_valu_shapes[] = {
#define DG_VS(path, mr, lpr) {path, mr, lpr},
    DG_SKINNY_VALU_CATALOGUE(DG_VS)
#undef DG_VS
};
const int k_mfma_paths[] = {
#define DG_MS(path) path,
    DG_SKINNY_MFMA_CATALOGUE(DG_MS)
#undef DG_MS
};
const int k_e2m1_mr[] = {
#define DG_ES(mr) mr,
    DG_SKINNY_E2M1_CATALOGUE(DG_ES)
#undef DG_ES
};

// Registers, LDS and occupancy of the compiled variants, as the compiler
// reported them when the library was built.
struct ResRow {
    int fam, a0, a1, a2, a3, a4, a5, a6, a7, vgpr, agpr, lds, occ, spill;
};
const ResRow k_res[] = {
#include "resources.inc"
};

const ResRow *find_res(int fam, int a0, int a1 = 0, int a2 = 0, int a3 = 0, int a4 = 0, int a5 = 0,
                       int a6 = 0, int a7 = 0)
{
    for (const ResRow &r : k_res)
        if (r.fam == fam && r.a0 == a0 && r.a1 == a1 && r.a2 == a2 && r.a3 == a3 && r.a4 == a4 &&
            r.a5 == a5 && r.a6 == a6 && r.a7 == a7)
            return &r;
    return nullptr;
}

const char *path_name(int p)
{
    switch (p) {
    case P_F16: return "f16";
    case P_BF16: return "bf16";
    case P_I8: return "i8";
    case P_MX: return "mx";
    default: return "e2m1";
    }
}

int elt_bytes(int t) { return (t == T_F16 || t == T_BF16) ? 2 : (t == T_I8 ? 1 : 4); }

// MFMA operations per clock per CU (2 per multiply-add): 16-bit 4096, int8 and
// the fp8 x fp4 block-scaled MFMA (the fp8 rate) 8192.
double mfma_ops_per_clk_cu(int path) { return (path == P_I8 || path == P_MX) ? 8192.0 : 4096.0; }

// Bytes per element of A and of B as stored.
double a_elt_bytes(int path) { return (path == P_I8 || path == P_MX) ? 1.0 : 2.0; }
double b_elt_bytes(int path)
{
    return path == P_I8 ? 1.0 : ((path == P_E2M1 || path == P_MX) ? 0.5 : 2.0);
}
// Block-scale bytes: e2m1 one fp16 per 32 codes of B; MX one byte per 32
// values of A and of B.
double scale_bytes(const Problem &pr)
{
    if (pr.path == P_E2M1) return (double)pr.N * (pr.K / 32) * 2;
    if (pr.path == P_MX) return (double)(pr.M + pr.N) * (pr.K / 32);
    return 0.0;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int round8(int x) { return (x + 7) & ~7; }

bool log_on()
{
    const char *e = std::getenv("DG_LOG");
    return e && std::atoi(e) >= 2;
}

// Occupancy from registers (512-entry unified file per lane) and LDS.
int waves_per_simd(int regs, int lds, int waves_wg, const dg_device_desc &d)
{
    int by_regs = std::min(d.max_waves_per_simd, d.vgpr_per_lane / std::max(8, round8(regs)));
    int wg_by_lds = lds > 0 ? d.lds_bytes_per_cu / lds : 64;
    int by_lds = wg_by_lds * waves_wg / d.simd_per_cu;
    return std::max(0, std::min(by_regs, by_lds));
}

// K splits to try: 1, 2, 4, ... while each slice keeps at least `min_slice`.
std::vector<int> split_choices(int64_t K, int unit, int min_slice, int force)
{
    std::vector<int> s;
    if (force > 0) {
        s.push_back(force);
        return s;
    }
    s.push_back(1);
    for (int v = 2; v <= 1024; v *= 2)
        if (K / v >= min_slice && K / v >= unit) s.push_back(v);
    return s;
}

// K splits for the streaming kernels: the powers of two, plus the counts that
// give the grid (grid_x column blocks per slice) about 3/4, one and two
// workgroups per CU.
std::vector<int> split_choices_grid(int64_t K, int unit, int min_slice, int force, int64_t grid_x, int cus)
{
    std::vector<int> s = split_choices(K, unit, min_slice, force);
    if (force > 0 || grid_x <= 0) return s;
    for (double f : {0.75, 1.0, 2.0}) {
        const int v = (int)std::ceil(f * cus / (double)grid_x);
        // (the slice as the kernel gets it: rounded up to the unit)
        const int64_t slice = (K + v - 1) / v + unit - 1 - ((K + v - 1) / v + unit - 1) % unit;
        if (v > 1 && v <= 1024 && slice >= min_slice && K / v >= unit &&
            std::find(s.begin(), s.end(), v) == s.end())
            s.push_back(v);
    }
    std::sort(s.begin(), s.end());
    return s;
}

// Slice length: a multiple of `unit`; the last slice takes what is left.
int slice_len(int64_t K, int S, int unit) { return (int)round_up(ceil_div(K, S), unit); }

void schedule(int64_t slice, int step, int &k_main, int &n_main, int &k_tail, int &n_tail)
{
    k_main = step;
    n_main = (int)(slice / step);
    k_tail = (int)(slice - (int64_t)n_main * step);
    n_tail = k_tail ? 1 : 0;
}

double clk_per_us(const dg_device_desc &d) { return d.clock_ghz * 1e3; }

double hbm_us(double bytes, const dg_device_desc &d) { return bytes / (d.hbm_gbps * 1e3); }

// Launch cost: the probe's empty launch when measured.
double launch_us(const dg_device_desc &d) { return d.launch_us > 0 ? d.launch_us : 2.0; }

// MFMA operations per microsecond per CU: the published rate (mfma_ops_per_clk_cu
// at the peak clock), or the probe's sustained fp16 rate (int8 and the fp8
// block-scaled MFMA at twice it).
double published_mfma_cu_us(int path, const dg_device_desc &d) { return mfma_ops_per_clk_cu(path) * clk_per_us(d); }
double probed_mfma_cu_us(int path, const dg_device_desc &d)
{
    if (d.mfma_tflops_f16 <= 0) return published_mfma_cu_us(path, d);
    const double f16 = d.mfma_tflops_f16 * 1e6 / d.cu_count;
    return (path == P_I8 || path == P_MX) ? 2 * f16 : f16;
}

// LDS bytes a CU reads per clock: two bytes per bank, the bank count being twice
// the probe's full-serialisation stride (64 banks on gfx950; fragment reads
// reach about that rate).
double lds_bytes_per_clk(const dg_device_desc &d)
{
    const int stride = d.lds_conflict_stride_words > 0 ? d.lds_conflict_stride_words : 32;
    return 2.0 * 2 * stride;
}

// Last-level cache: operands larger than it are streamed from HBM.
double mall_bytes(const dg_device_desc &d) { return d.mall_bytes > 0 ? d.mall_bytes : 256.0 * 1024 * 1024; }

// Workspace bytes of a plan with S slices: the partial sums, with one more
// slice for the pad_k tail (which is then the only slice when the aligned
// part of K is empty).
int64_t plan_ws_bytes(const Problem &pr, int S)
{
    if (pr.k_pad) return ((pr.K == 0 ? 0 : S) + 1) * pr.M * pr.N * 4;
    return S > 1 ? (int64_t)S * pr.M * pr.N * 4 : 0;
}

// The problem's workspace limit rules this plan out (a forced split is kept:
// the caller reports it).
bool over_ws_limit(const Problem &pr, int S, const dg_plan_opts &o)
{
    return pr.ws_limit >= 0 && !o.force_split_k && plan_ws_bytes(pr, S) > pr.ws_limit;
}

}  // namespace

double roofline_us(const Problem &pr, const dg_device_desc &d)
{
    double bytes = pr.M * pr.K * a_elt_bytes(pr.path) + pr.K * pr.N * b_elt_bytes(pr.path) +
                   pr.M * pr.N * elt_bytes(pr.out_type) + scale_bytes(pr);
    if (pr.beta_nz) bytes += pr.M * pr.N * elt_bytes(pr.out_type);
    const double flops = 2.0 * pr.M * pr.N * pr.K;
    const double t_mem = hbm_us(bytes, d);
    const double t_mfma = flops / (mfma_ops_per_clk_cu(pr.path) * d.cu_count * clk_per_us(d));
    return std::max(t_mem, t_mfma);
}

// ------------------------------------------------------------------ families
static void enum_tiled(const Problem &pr, const dg_device_desc &d, const dg_plan_opts &o, const EffTable *eff,
                       std::vector<Candidate> &out, int &enumerated, int &pruned, int &ws_pruned)
{
    const int KSUB = tiled_ksub(pr.path);
    const int lds_cap = std::min(d.lds_bytes_per_wg, o.lds_limit_bytes > 0 ? o.lds_limit_bytes : 1 << 30);
    const int occ_need = std::max(1, (int)std::ceil(o.target_occupancy * d.max_waves_per_simd - 1e-9));
    const int nshapes = (int)(sizeof(k_tiled_shapes) / sizeof(k_tiled_shapes[0]));
    for (int id = 0; id < nshapes; ++id) {
        const TiledShape &s = k_tiled_shapes[id];
        if (s.path != pr.path || s.b_kmajor != pr.b_kmajor) continue;
        const int BKE = tiled_bk_elems(pr.path) * s.kr;   // the variant's K step (K_tile)
        const int waves = s.wm * s.wn, NT = waves * 64;
        const int FM = s.bm / s.wm / 32, FN = s.bn / s.wn / 32;
        // registers (per lane): accumulators, staging, fragments, addressing
        const int acc = FM * FN * 16;
        int stage = s.bm * 8 * s.kr / NT * 4;
        if (pr.path == P_MX) stage = s.bm * 16 / NT * 4 + s.bn * 8 / NT * 4 + (FM + FN) * 2;
        else if (pr.path == P_E2M1) stage += ceil_div(s.bn * 2, NT) * 5;
        else if (s.b_kmajor) stage += s.bn * 8 * s.kr / NT * 4;
        else stage += (int)ceil_div(s.bn, NT) * 32 * s.kr;
        const int other = stage + (FM + FN) * 4 * 2 + 40;
        int vgpr, agpr;
        if (acc + other <= 256) { vgpr = acc + other; agpr = 0; }
        else { vgpr = other; agpr = acc; }
        int lds = tiled_lds_bytes(s.path, s.bm, s.bn, s.wm, s.wn, s.kr);
        if (const ResRow *r = find_res(F_TILED, s.path, s.b_kmajor, s.bm, s.bn, s.wm, s.wn, s.kr, s.ms)) {
            vgpr = r->vgpr;
            agpr = r->agpr;
            lds = r->lds;
        }
        const int occ = waves_per_simd(vgpr + agpr, lds, waves, d);

        const int min_slice = 4 * BKE;
        for (int S : split_choices(pr.K, BKE, min_slice, o.force_split_k)) {
            ++enumerated;
            // (MX slices start on whole steps: a step's four scales are one
            // aligned dword)
            const int unit = (pr.K >= (int64_t)S * BKE || pr.path == P_MX) ? BKE : KSUB;
            int k_slice = pr.K > 0 ? slice_len(pr.K, S, unit) : 0;
            const int S_eff = pr.K > 0 ? (int)ceil_div(pr.K, std::max(1, k_slice)) : 1;
            if (S_eff == 1) k_slice = (int)pr.K;   // one slice: exactly K, tail included
            // constraints
            const char *why = nullptr;
            if (lds > lds_cap) why = "LDS over budget";
            else if (agpr > 256 || vgpr > 256) why = "registers over budget";
            else if (occ < occ_need) why = "occupancy below target";
            else if (o.force_m_tile && o.force_m_tile != s.bm) why = "forced M tile";
            else if (o.force_n_tile && o.force_n_tile != s.bn) why = "forced N tile";
            else if (o.force_k_tile && o.force_k_tile != BKE) why = "forced K tile";
            else if (o.force_waves && o.force_waves != waves) why = "forced wave count";
            else if (o.force_mfma && o.force_mfma != s.ms) why = "forced MFMA block";
            else if (S_eff != S && !o.force_split_k) why = "split collapses";
            else if (over_ws_limit(pr, S_eff, o)) {
                why = "workspace over the limit";
                ++ws_pruned;
            }
            if (why) {
                ++pruned;
                if (log_on())
                    std::fprintf(stderr, "[dg] prune tiled %dx%d w%dx%d S=%d: %s\n", s.bm, s.bn, s.wm,
                                 s.wn, S, why);
                continue;
            }
            Candidate c{};
            c.family = F_TILED;
            c.kernel_id = id;
            c.unit = DG_UNIT_MFMA;
            c.mfma_m = s.ms; c.mfma_n = s.ms; c.mfma_k = s.ms == 16 ? 2 * KSUB : KSUB;
            c.m_tile = s.bm; c.n_tile = s.bn; c.waves = waves;
            c.split_k = S_eff; c.k_slice = k_slice;
            schedule(k_slice, BKE, c.k_main, c.n_main, c.k_tail, c.n_tail);
            c.lds = lds; c.vgpr = vgpr; c.agpr = agpr; c.waves_per_simd = occ;
            const int64_t tiles = ceil_div(pr.M, s.bm) * ceil_div(pr.N, s.bn);
            c.grid_x = (int)tiles;
            c.grid_y = S_eff;
            c.ws_bytes = S_eff > 1 ? (int64_t)S_eff * pr.M * pr.N * 4 : 0;
            // ---- cost model (microseconds)
            const double cpu = clk_per_us(d);
            const int wg_per_cu = std::max(1, occ * d.simd_per_cu / waves);
            const int64_t wgs = tiles * S_eff;
            const int64_t rounds = ceil_div(wgs, (int64_t)d.cu_count * wg_per_cu);
            const int W = (int)std::min<int64_t>(wg_per_cu, ceil_div(wgs, d.cu_count));
            // MFMA time of one K step: with a measured efficiency for this variant
            // (the probe's calibration), the probed MFMA rate times it; without,
            // the published rate times the built-in fraction (catalogue.h).  The
            // LDS and L2 terms only matter for variants that are not MFMA-bound.
            char nm[64];
            std::snprintf(nm, sizeof nm, "tiled_%s_%s_%dx%d_w%dx%d_k%d%s", path_name(pr.path),
                          pr.b_kmajor ? "k" : "n", s.bm, s.bn, s.wm, s.wn, BKE, s.ms == 16 ? "_m16" : "");
            const double step_ops = 2.0 * s.bm * s.bn * BKE;
            double t_mfma, round_us = -1;
            const auto hit = eff ? eff->eff.find(nm) : std::unordered_map<std::string, double>::const_iterator();
            if (eff && hit != eff->eff.end() && hit->second > 0) {
                t_mfma = step_ops / (probed_mfma_cu_us(pr.path, d) * hit->second);
                const auto r = eff->round_us.find(nm);
                if (r != eff->round_us.end() && r->second >= 0) round_us = r->second;
            } else {
                t_mfma = step_ops / (published_mfma_cu_us(pr.path, d) *
                                     tiled_step_efficiency(s.path, s.bm, s.bn, waves, s.kr));
            }
            const double stage = tiled_stage_bytes(s.path, s.bm, s.bn, s.kr);
            const double t_lds = (waves * (BKE / KSUB) * (FM + FN) * 1024.0 + stage) / lds_bytes_per_clk(d) / cpu;
            const double t_l2 = stage / 64.0 / cpu;
            // A K step waits for loads issued one step earlier.  When an operand is
            // streamed with almost no reuse across workgroups (one or two tile rows
            // or columns), or the operands do not fit the last-level cache, those
            // loads come from HBM and the step is bound by DRAM latency (~1.7 us);
            // otherwise mostly by L2 latency (~0.33 us).
            const int64_t tm = ceil_div(pr.M, s.bm), tn = ceil_div(pr.N, s.bn);
            const double op_bytes = pr.M * pr.K * a_elt_bytes(pr.path) + pr.K * pr.N * b_elt_bytes(pr.path);
            const double lat = ((tm <= 2 || tn <= 2 || op_bytes > mall_bytes(d)) ? 4000.0 : 800.0) / cpu;
            const double per_step = std::max(W * std::max(t_mfma, std::max(t_lds, t_l2)), lat);
            const double steps = ceil_div(std::max(k_slice, 1), BKE);
            const double t_comp = rounds * steps * per_step;
            double floor_bytes = pr.M * pr.K * a_elt_bytes(pr.path) + pr.K * pr.N * b_elt_bytes(pr.path) +
                                 scale_bytes(pr);
            const double out_bytes = (double)pr.M * pr.N * elt_bytes(pr.out_type) * (pr.beta_nz ? 2 : 1);
            double est;
            if (round_us >= 0) {
                // measured: each round of workgroups costs its fixed time (entry,
                // epilogue with its stores, launch share) plus its K steps
                est = std::max(rounds * round_us + t_comp, hbm_us(floor_bytes + out_bytes, d));
            } else {
                // the epilogue stores after the K loop, at about 70 % of HBM bandwidth
                est = std::max(t_comp, hbm_us(floor_bytes, d)) + hbm_us(out_bytes, d) / 0.7 + launch_us(d);
            }
            // a K split: the tiles' epilogues write fp32 partial sums in place of
            // the output (measured to cost about what the output's stores do),
            // and the reduction reads them and writes the output: one more
            // launch
            if (S_eff > 1) est += hbm_us((double)S_eff * pr.M * pr.N * 4 + out_bytes, d) + launch_us(d);
            c.est_us = est;
            c.roof_us = roofline_us(pr, d);
            c.name = nm;
            out.push_back(c);
        }
    }
}

// Skinny families: a requested split S whose rounded slices give fewer slices
// (S_eff) is kept as a plan with S_eff slices (the streaming kernels take any
// slice count).
static void enum_skinny(const Problem &pr, const dg_device_desc &d, const dg_plan_opts &o,
                        std::vector<Candidate> &out, int &enumerated, int &pruned, int &ws_pruned)
{
    if (o.force_m_tile || o.force_k_tile || o.force_waves || o.force_mfma) return;  // tiled-only options
    // force_n_tile picks the streaming kernels' columns per workgroup
    auto n_ok = [&](int n_tile) { return o.force_n_tile == 0 || o.force_n_tile == n_tile; };
    const int lds_cap = std::min(d.lds_bytes_per_wg, o.lds_limit_bytes > 0 ? o.lds_limit_bytes : 1 << 30);
    const int occ_need = std::max(1, (int)std::ceil(o.target_occupancy * d.max_waves_per_simd - 1e-9));
    const double cpu = clk_per_us(d);
    const double out_bytes = (double)pr.M * pr.N * elt_bytes(pr.out_type) * (pr.beta_nz ? 2 : 1);

    // `cols_per_wave`: columns one wave streams; waves past N idle, and a partly
    // filled wave counts for the share of its lanes that have columns.
    // `by_wg`: the stream's rate is set by its workgroups rather than its waves
    // (the long-K kernels, whose workgroups each keep deep double-buffered loads
    // in flight).  Measured on MI355X (bf16, N = 4096, K = 131072): HBM is
    // saturated from about 3/4 of the CUs with one workgroup each; a grid
    // between one and two workgroups per CU leaves the CUs with two as the
    // critical path (the time of a full second round); splits beyond that only
    // add partial sums.
    auto finish = [&](Candidate &c, double b_bytes, double valu_lane_ops, int cols_per_wave, bool by_wg = false) {
        double eff;
        if (by_wg) {
            const double wgs = (double)c.grid_x * c.grid_y;
            const double rounds = std::ceil(wgs / d.cu_count);
            eff = wgs <= d.cu_count ? std::min(1.0, wgs / (0.75 * d.cu_count)) : wgs / (rounds * d.cu_count);
            // the share of the workgroups' columns that exist (four waves each)
            eff *= std::min(1.0, (double)pr.N / ((double)c.grid_x * 4 * cols_per_wave));
            // waves of 64 columns (128-byte row pieces) stream about 5 % slower
            // than wider ones (measured: bf16, M = 1, N = 4096, K = 131072,
            // 173-179 us at 192-512 workgroups against 169 us with 128 columns)
            if (cols_per_wave < 128) eff *= 0.95;
        } else {
            const double waves_active = c.grid_y * (double)pr.N / cols_per_wave;
            eff = std::min(1.0, waves_active / (d.cu_count * 8.0));
        }
        const double t_mem = hbm_us(b_bytes, d) / (0.92 * std::max(eff, 1e-3));
        const double t_valu = valu_lane_ops / (d.cu_count * 64.0 * cpu);
        double est = std::max(t_mem, t_valu) + hbm_us(out_bytes, d) + launch_us(d);
        if (c.split_k > 1) est += hbm_us((double)c.split_k * pr.M * pr.N * 4 * 2, d) + launch_us(d);
        c.est_us = est;
        c.roof_us = roofline_us(pr, d);
    };

    // VALU over a row-major 16-bit B
    if ((pr.path == P_F16 || pr.path == P_BF16) && !pr.b_kmajor && pr.M <= 8 &&
        o.unit != DG_UNIT_MFMA) {
        const int nv = (int)(sizeof(k_valu_shapes) / sizeof(k_valu_shapes[0]));
        for (int id = 0; id < nv; ++id) {
            const ValuShape &s = k_valu_shapes[id];
            if (s.path != pr.path || s.mr < pr.M || (s.mr > 1 && s.mr / 2 >= pr.M)) continue;
            const int rpi = 64 / s.lpr;
            const int wcols = s.lpr * 8;
            if (!n_ok(4 * wcols)) continue;
            for (int S : split_choices_grid(pr.K, 16, 64, o.force_split_k, ceil_div(pr.N, 4 * wcols), d.cu_count)) {
                ++enumerated;
                int k_slice = pr.K > 0 ? slice_len(pr.K, S, 16) : 0;
                const int S_eff = pr.K > 0 ? (int)ceil_div(pr.K, std::max(1, k_slice)) : 1;
                if (S_eff == 1) k_slice = (int)pr.K;
                int lds = SKINNY_A_LDS;
                int regs = 40 + s.mr * 8 + 8 * 4 + 16;
                if (const ResRow *r = find_res(F_SKINNY_VALU, s.path, s.mr, s.lpr)) {
                    regs = r->vgpr + r->agpr;
                    lds = r->lds;
                }
                const int occ = waves_per_simd(regs, lds, 4, d);
                const char *why = nullptr;
                if ((int64_t)k_slice * s.mr * 2 > SKINNY_A_LDS) why = "A slice over LDS staging";
                else if (lds > lds_cap) why = "LDS over budget";
                else if (occ < occ_need) why = "occupancy below target";
                else if (o.force_path == DG_PATH_TILED) why = "forced tiled path";
                else if (over_ws_limit(pr, S_eff, o)) {
                    why = "workspace over the limit";
                    ++ws_pruned;
                }
                if (why) {
                    ++pruned;
                    continue;
                }
                Candidate c{};
                c.family = F_SKINNY_VALU;
                c.kernel_id = id;
                c.unit = DG_UNIT_VALU;
                c.m_tile = s.mr; c.n_tile = 4 * wcols; c.waves = 4;
                c.split_k = S_eff; c.k_slice = k_slice;
                schedule(k_slice, 8 * rpi, c.k_main, c.n_main, c.k_tail, c.n_tail);
                if (c.k_tail) { c.n_tail = c.k_tail / rpi + (c.k_tail % rpi ? 1 : 0); c.k_tail = rpi; }
                c.lds = lds; c.vgpr = regs; c.agpr = 0; c.waves_per_simd = occ;
                c.grid_x = (int)ceil_div(pr.N, 4 * wcols);
                c.grid_y = S_eff;
                c.ws_bytes = S_eff > 1 ? (int64_t)S_eff * pr.M * pr.N * 4 : 0;
                finish(c, (double)pr.K * pr.N * 2 + pr.M * pr.K * 2.0,
                       (double)s.mr * pr.K * pr.N * 1.3 + (double)pr.K * pr.N, wcols, true);
                char nm[64];
                std::snprintf(nm, sizeof nm, "skinny_valu_%s_mr%d_lpr%d", path_name(pr.path), s.mr, s.lpr);
                c.name = nm;
                out.push_back(c);
            }
        }
    }
    // MFMA over a row-major 16-bit B, M <= 16
    if ((pr.path == P_F16 || pr.path == P_BF16) && !pr.b_kmajor && pr.M <= 16 &&
        o.unit != DG_UNIT_VALU) {
        const int nm_ = (int)(sizeof(k_mfma_paths) / sizeof(k_mfma_paths[0]));
        for (int id = 0; id < nm_; ++id) {
            if (k_mfma_paths[id] != pr.path || !n_ok(512)) continue;
            for (int S : split_choices_grid(pr.K, 32, 256, o.force_split_k, ceil_div(pr.N, 512), d.cu_count)) {
                ++enumerated;
                int k_slice = pr.K > 0 ? slice_len(pr.K, S, 32) : 0;
                const int S_eff = pr.K > 0 ? (int)ceil_div(pr.K, std::max(1, k_slice)) : 1;
                if (S_eff == 1) k_slice = (int)pr.K;
                int vg = 64, ag = 48;
                if (const ResRow *r = find_res(F_SKINNY_MFMA, pr.path)) {
                    vg = r->vgpr;
                    ag = r->agpr;
                }
                const int occ = waves_per_simd(vg + ag, 0, 4, d);
                const char *why = nullptr;
                if (occ < occ_need) why = "occupancy below target";
                else if (o.force_path == DG_PATH_TILED) why = "forced tiled path";
                else if (over_ws_limit(pr, S_eff, o)) {
                    why = "workspace over the limit";
                    ++ws_pruned;
                }
                if (why) {
                    ++pruned;
                    continue;
                }
                Candidate c{};
                c.family = F_SKINNY_MFMA;
                c.kernel_id = id;
                c.unit = DG_UNIT_MFMA;
                c.mfma_m = 16; c.mfma_n = 16; c.mfma_k = 32;
                c.m_tile = 16; c.n_tile = 512; c.waves = 4;
                c.split_k = S_eff; c.k_slice = k_slice;
                schedule(k_slice, 32, c.k_main, c.n_main, c.k_tail, c.n_tail);
                c.lds = 0; c.vgpr = vg; c.agpr = ag; c.waves_per_simd = occ;
                c.grid_x = (int)ceil_div(pr.N, 512);
                c.grid_y = S_eff;
                c.ws_bytes = S_eff > 1 ? (int64_t)S_eff * pr.M * pr.N * 4 : 0;
                finish(c, (double)pr.K * pr.N * 2 + 16.0 * pr.K * 2 * c.grid_x,
                       (double)pr.K * pr.N * 0.6, 128, true);
                char nm[64];
                std::snprintf(nm, sizeof nm, "skinny_mfma_%s", path_name(pr.path));
                c.name = nm;
                out.push_back(c);
            }
        }
    }
    // e2m1 weights, small M (vector dot products)
    if (pr.path == P_E2M1 && pr.M <= 8 && o.unit != DG_UNIT_MFMA) {
        const int ne = (int)(sizeof(k_e2m1_mr) / sizeof(k_e2m1_mr[0]));
        for (int id = 0; id < ne; ++id) {
            const int mr = k_e2m1_mr[id];
            if (mr < pr.M || (mr > 1 && mr / 2 >= pr.M) || !n_ok(16)) continue;
            for (int S : split_choices(pr.K, 32, 2048, o.force_split_k)) {
                ++enumerated;
                int k_slice = pr.K > 0 ? slice_len(pr.K, S, 32) : 0;
                const int S_eff = pr.K > 0 ? (int)ceil_div(pr.K, std::max(1, k_slice)) : 1;
                if (S_eff == 1) k_slice = (int)pr.K;
                int vg = 48;
                if (const ResRow *r = find_res(F_SKINNY_E2M1, mr)) vg = r->vgpr + r->agpr;
                int lds_e = E2M1_A_LDS;
                if (const ResRow *r = find_res(F_SKINNY_E2M1, mr)) lds_e = r->lds;
                const int occ = waves_per_simd(vg, lds_e, 4, d);
                const char *why = nullptr;
                if ((int64_t)k_slice * mr * 2 > E2M1_A_LDS) why = "A slice over LDS staging";
                else if (lds_e > lds_cap) why = "LDS over budget";
                else if (occ < occ_need) why = "occupancy below target";
                else if (o.force_path == DG_PATH_TILED) why = "forced tiled path";
                else if (over_ws_limit(pr, S_eff, o)) {
                    why = "workspace over the limit";
                    ++ws_pruned;
                }
                if (why) {
                    ++pruned;
                    continue;
                }
                Candidate c{};
                c.family = F_SKINNY_E2M1;
                c.kernel_id = id;
                c.unit = DG_UNIT_VALU;
                c.m_tile = mr; c.n_tile = 16; c.waves = 4;
                c.split_k = S_eff; c.k_slice = k_slice;
                schedule(k_slice, 32 * 64, c.k_main, c.n_main, c.k_tail, c.n_tail);
                if (c.k_tail) { c.n_tail = 1; }
                c.lds = lds_e; c.vgpr = vg; c.agpr = 0; c.waves_per_simd = occ;
                c.grid_x = (int)ceil_div(pr.N, 16);
                c.grid_y = S_eff;
                c.ws_bytes = S_eff > 1 ? (int64_t)S_eff * pr.M * pr.N * 4 : 0;
                finish(c, (double)pr.K * pr.N * 0.5 + (double)pr.N * (pr.K / 32) * 2 + pr.M * pr.K * 2.0,
                       (double)pr.N * (pr.K / 32) * (24.0 + 16.0 * mr), 4);
                char nm[64];
                std::snprintf(nm, sizeof nm, "skinny_e2m1_mr%d", mr);
                c.name = nm;
                out.push_back(c);
            }
        }
    }
}

static bool dominates(const Candidate &a, const Candidate &b)
{
    const int ra = a.vgpr + a.agpr, rb = b.vgpr + b.agpr;
    const bool le = a.est_us <= b.est_us && a.lds <= b.lds && ra <= rb;
    const bool lt = a.est_us < b.est_us || a.lds < b.lds || ra < rb;
    return le && lt;
}

static bool better(const Candidate &a, const Candidate &b)
{
    if (a.est_us != b.est_us) return a.est_us < b.est_us;
    if (a.lds != b.lds) return a.lds < b.lds;
    if (a.m_tile != b.m_tile) return a.m_tile < b.m_tile;
    if (a.n_tile != b.n_tile) return a.n_tile < b.n_tile;
    if (a.k_main != b.k_main) return a.k_main < b.k_main;
    if (a.split_k != b.split_k) return a.split_k < b.split_k;
    return a.name < b.name;
}

PlanResult plan_problem(const Problem &pr, const dg_device_desc &d, const dg_plan_opts &o, const EffTable *eff)
{
    PlanResult res;
    std::vector<Candidate> all;
    const bool want_tiled = o.force_path != DG_PATH_SKINNY && o.unit != DG_UNIT_VALU;
    const bool want_skinny = o.force_path != DG_PATH_TILED;
    if (o.unit == DG_UNIT_VALU && o.force_path == DG_PATH_TILED) {
        res.status = DG_ERR_CONFLICT;
        res.message = "conflicting compute units: the tiled path runs on MFMA, VALU was requested";
        return res;
    }
    if (o.force_path == DG_PATH_SKINNY && (o.force_m_tile || o.force_k_tile || o.force_waves || o.force_mfma)) {
        res.status = DG_ERR_CONFLICT;
        res.message = "forced M tile, K step, waves and MFMA block apply to the tiled path, the skinny path was forced";
        return res;
    }
    if (want_tiled) enum_tiled(pr, d, o, eff, all, res.enumerated, res.pruned, res.ws_pruned);
    if (want_skinny) enum_skinny(pr, d, o, all, res.enumerated, res.pruned, res.ws_pruned);
    if (all.empty() && res.ws_pruned > 0) {
        res.status = DG_ERR_WORKSPACE;
        char m[160];
        std::snprintf(m, sizeof m, "no plan's partial sums fit the %lld-byte workspace limit "
                      "(%d candidates pruned by it)", (long long)pr.ws_limit, res.ws_pruned);
        res.message = m;
        return res;
    }
    if (all.empty()) {
        res.status = DG_ERR_NO_CANDIDATE;
        char m[160];
        std::snprintf(m, sizeof m, "No valid candidate found after pruning (%d enumerated, %d pruned)",
                      res.enumerated, res.pruned);
        res.message = m;
        return res;
    }
    std::vector<Candidate> par;
    for (size_t i = 0; i < all.size(); ++i) {
        bool dom = false;
        for (size_t j = 0; j < all.size() && !dom; ++j)
            if (j != i && dominates(all[j], all[i])) dom = true;
        if (!dom) par.push_back(all[i]);
    }
    std::sort(par.begin(), par.end(), better);
    if (log_on()) {
        std::fprintf(stderr, "[dg] M=%lld N=%lld K=%lld path=%s: %d enumerated, %d pruned, %zu feasible, %zu Pareto\n",
                     (long long)pr.M, (long long)pr.N, (long long)pr.K, path_name(pr.path), res.enumerated,
                     res.pruned, all.size(), par.size());
        for (const Candidate &c : par)
            std::fprintf(stderr, "[dg]   %-34s S=%-4d est %.2f us lds %d regs %d\n", c.name.c_str(),
                         c.split_k, c.est_us, c.lds, c.vgpr + c.agpr);
    }
    res.status = DG_OK;
    res.pareto = par;
    return res;
}

void fill_info(const Candidate &c, dg_plan_info *o)
{
    std::memset(o, 0, sizeof *o);
    o->path = c.family == F_TILED ? DG_PATH_TILED : DG_PATH_SKINNY;
    o->unit = c.unit;
    o->mfma_m = c.mfma_m; o->mfma_n = c.mfma_n; o->mfma_k = c.mfma_k;
    o->m_tile = c.m_tile; o->n_tile = c.n_tile;
    o->k_main = c.k_main; o->n_main = c.n_main; o->k_tail = c.k_tail; o->n_tail = c.n_tail;
    o->split_k = c.split_k + (c.k_pad ? 1 : 0); o->k_slice = c.k_slice;
    o->waves_per_wg = c.waves;
    o->lds_bytes = c.lds; o->vgpr_est = c.vgpr; o->agpr_est = c.agpr;
    o->waves_per_simd = c.waves_per_simd;
    o->grid = c.grid_x * c.grid_y;
    o->workspace_bytes = c.ws_bytes;
    o->est_us = c.est_us;
    o->est_roof_fraction = c.est_us > 0 ? c.roof_us / c.est_us : 0;
    o->kernel_id = c.family * 1000 + c.kernel_id;
    std::snprintf(o->kernel_name, sizeof o->kernel_name, "%s", c.name.c_str());
}

}  // namespace dg
