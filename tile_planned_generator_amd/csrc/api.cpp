// api.cpp - the C ABI (include/dg.h): validation, plan cache, dispatch.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/dg.h"
#include "catalogue.h"
#include "dg_args.h"
#include "launch.h"
#include "planner.h"

using namespace dg;

struct dg_handle_s {
    dg_device_desc desc;
    int device;   // -1: offline (planner only)
    EffTable eff;  // measured tiled-variant efficiencies (dg_load_device_json)
    std::unordered_map<std::string, Candidate> cache;
    uint64_t *clk = nullptr;    // stage clock buffer (dg_set_stage_clock), or null
    int64_t clk_entries = 0;
};

namespace {

thread_local std::string g_err;
std::mutex g_live_mu;
std::set<const void *> g_live;

dg_status fail(dg_status s, const std::string &msg)
{
    g_err = msg;
    return s;
}

dg_status ok()
{
    return DG_OK;
}

bool is_live(dg_handle_t h)
{
    std::lock_guard<std::mutex> lk(g_live_mu);
    return h && g_live.count(h);
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elt_of(int32_t t)
{
    switch (t) {
    case DG_F16: return T_F16;
    case DG_BF16: return T_BF16;
    case DG_F32: return T_F32;
    case DG_I32: return T_I32;
    case DG_I8: return T_I8;
    default: return -1;
    }
}

int elt_size(int e) { return (e == T_F16 || e == T_BF16) ? 2 : (e == T_I8 ? 1 : 4); }

// Validate a problem description and build the planner's view of it.
dg_status describe(int64_t M, int64_t N, int64_t K, const dg_dtypes *dt, const dg_layouts *lay,
                   int32_t group_k, int32_t epi_kind, int beta_nz, int pad_k, Problem &pr)
{
    if (!dt) return fail(DG_ERR_INVALID_ARG, "dtypes is NULL");
    if (M < 0 || N < 0 || K < 0) return fail(DG_ERR_INVALID_ARG, "negative size");
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return fail(DG_ERR_UNSUPPORTED, "sizes above 2^31-1 are not supported");
    int path;
    if (dt->a == DG_F16 && dt->b == DG_F16) path = P_F16;
    else if (dt->a == DG_BF16 && dt->b == DG_BF16) path = P_BF16;
    else if (dt->a == DG_I8 && dt->b == DG_I8) path = P_I8;
    else if (dt->a == DG_F16 && dt->b == DG_E2M1) path = P_E2M1;
    else if (dt->a == DG_F8E4M3 && dt->b == DG_E2M1) path = P_MX;
    else return fail(DG_ERR_UNSUPPORTED, "unsupported (a, b) dtype pair");
    const bool fp4b = path == P_E2M1 || path == P_MX;
    const bool is_int = path == P_I8;
    if (dt->compute != (is_int ? DG_I32 : DG_F32))
        return fail(DG_ERR_UNSUPPORTED, is_int ? "int8 inputs accumulate in I32" : "16-bit, e2m1 and MX inputs accumulate in F32");
    if (path == P_MX && beta_nz) return fail(DG_ERR_UNSUPPORTED, "the MX path has no beta * D term");
    if (epi_kind < DG_EPI_NONE || epi_kind > DG_EPI_REQUANT_F16)
        return fail(DG_ERR_INVALID_ARG, "unknown epilogue kind");
    const bool rq = epi_kind == DG_EPI_REQUANT_I8 || epi_kind == DG_EPI_REQUANT_F16;
    if (is_int) {
        const int want = epi_kind == DG_EPI_NONE ? DG_I32 : (epi_kind == DG_EPI_REQUANT_I8 ? DG_I8 : DG_F16);
        if (!(epi_kind == DG_EPI_NONE || rq))
            return fail(DG_ERR_UNSUPPORTED, "the int8 path supports the NONE and requantise epilogues");
        if (dt->c != want) return fail(DG_ERR_UNSUPPORTED, "output dtype does not match the int8 epilogue");
        if (rq && beta_nz) return fail(DG_ERR_INVALID_ARG, "requantise epilogues need beta == 0");
    } else {
        if (rq) return fail(DG_ERR_UNSUPPORTED, "requantise epilogues need the int8 path");
        const int own = path == P_BF16 ? DG_BF16 : DG_F16;
        if (dt->c != own && dt->c != DG_F32)
            return fail(DG_ERR_UNSUPPORTED, "output dtype must be the input's 16-bit type or F32");
    }
    // layouts
    dg_layouts L{};
    if (lay) L = *lay;
    else L.b = fp4b ? DG_COL_MAJOR : DG_ROW_MAJOR;
    if (L.a != DG_ROW_MAJOR) return fail(DG_ERR_UNSUPPORTED, "A must be row-major");
    if (L.b != DG_ROW_MAJOR && L.b != DG_COL_MAJOR) return fail(DG_ERR_INVALID_ARG, "unknown B layout");
    if (fp4b && L.b != DG_COL_MAJOR)
        return fail(DG_ERR_UNSUPPORTED, "e2m1 B must be column-major (N x K, K contiguous)");
    const int64_t lda = L.lda ? L.lda : K;
    const int64_t ldb = L.ldb ? L.ldb : (L.b == DG_ROW_MAJOR ? N : K);
    const int64_t ldc = L.ldc ? L.ldc : N;
    const int64_t ldd = L.ldd ? L.ldd : N;
    if (lda < K || ldb < (L.b == DG_ROW_MAJOR ? N : K) || ldc < N || ldd < N)
        return fail(DG_ERR_INVALID_ARG, "a leading dimension is smaller than the matrix");
    // alignment: K in whole MFMA steps, rows on 16-byte boundaries
    const int ksub = path == P_MX ? 64 : ((path == P_I8 || path == P_E2M1) ? 32 : 16);
    int64_t k_pad = 0;
    if (K % ksub) {
        if (!pad_k)
            return fail(DG_ERR_ALIGNMENT, "K dimension not aligned to the MFMA depth (" + std::to_string(ksub) +
                                              "); set pad_k to add the tail separately");
        if (path == P_E2M1) return fail(DG_ERR_UNSUPPORTED, "e2m1 needs K in whole 32-element groups");
        if (path == P_MX) return fail(DG_ERR_UNSUPPORTED, "the MX path needs K in whole 64-element MFMA steps");
        k_pad = K % ksub;
    }
    if (fp4b && group_k != 32) return fail(DG_ERR_UNSUPPORTED, "e2m1 and MX need group_k == 32");
    const int esz = (path == P_I8 || path == P_MX) ? 1 : 2;
    if (K > 0) {   // with K == 0 neither A nor B is read
        if ((lda * esz) % 16) return fail(DG_ERR_ALIGNMENT, "lda is not a multiple of 16 bytes");
        if (fp4b) {
            if (ldb % 32) return fail(DG_ERR_ALIGNMENT, "ldb (codes) is not a multiple of 32");
        } else if ((ldb * esz) % 16) {
            return fail(DG_ERR_ALIGNMENT, "ldb is not a multiple of 16 bytes");
        }
    }
    pr.M = M;
    pr.N = N;
    pr.K = K - k_pad;   // the aligned part; pad_k adds the rest as one more partial slice
    pr.k_pad = k_pad;
    pr.path = path;
    pr.b_kmajor = L.b == DG_COL_MAJOR;
    pr.out_type = elt_of(dt->c);
    pr.epi = epi_kind;
    pr.beta_nz = beta_nz;
    return DG_OK;
}

dg_plan_opts opts_or_default(const dg_plan_opts *o)
{
    dg_plan_opts d{};
    if (o) d = *o;
    if (d.target_occupancy <= 0.f) d.target_occupancy = 0.125f;
    return d;
}

std::string cache_key(const Problem &p, const dg_plan_opts &o)
{
    char k[256];
    std::snprintf(k, sizeof k, "%lld,%lld,%lld+%lld,%lld,%d,%d,%d,%d,%d|%d,%d,%d,%d,%d,%d,%d,%.4f,%d,%d,%d",
                  (long long)p.M, (long long)p.N, (long long)p.K, (long long)p.k_pad, (long long)p.ws_limit,
                  p.path, p.b_kmajor,
                  p.out_type, p.epi,
                  p.beta_nz, o.force_m_tile, o.force_n_tile, o.force_k_tile, o.force_split_k, o.force_path,
                  o.unit, o.lds_limit_bytes, o.target_occupancy, o.pad_k, o.force_waves, o.force_mfma);
    return k;
}

// pad_k: the plan of the aligned part, plus one partial slice for the K tail;
// the partials are then reduced, with the epilogue, by the split-K reduction.
void add_tail(const Problem &pr, const dg_device_desc &d, Candidate &c)
{
    if (!pr.k_pad) return;
    c.k_pad = (int)pr.k_pad;
    if (pr.K == 0) {   // no aligned part: the tail is the only slice, no main launch
        c.split_k = 0;
        c.grid_y = 0;
    }
    const int64_t slices = c.split_k + 1;
    c.ws_bytes = slices * pr.M * pr.N * 4;
    // the tail kernel and the reduce: partials written and read once, two launches
    c.est_us += (double)(slices + 1) * pr.M * pr.N * 4 / (d.hbm_gbps * 1e3) + 2 * 4.0;
}

dg_status plan_cached(dg_handle_t h, const Problem &pr, const dg_plan_opts &o, Candidate &out)
{
    if (o.pad_k < 0 || o.pad_k > 1) return fail(DG_ERR_INVALID_ARG, "pad_k is 0 or 1");
    if (o.unit < DG_UNIT_AUTO || o.unit > DG_UNIT_VALU) return fail(DG_ERR_INVALID_ARG, "unknown unit");
    if (o.force_path < DG_PATH_AUTO || o.force_path > DG_PATH_SKINNY)
        return fail(DG_ERR_INVALID_ARG, "unknown path");
    if (o.force_split_k < 0 || o.force_m_tile < 0 || o.force_n_tile < 0 || o.force_k_tile < 0 ||
        o.force_waves < 0 || (o.force_mfma != 0 && o.force_mfma != 16 && o.force_mfma != 32) ||
        o.lds_limit_bytes < 0 || o.target_occupancy > 1.0f)
        return fail(DG_ERR_INVALID_ARG, "invalid planner option");
    const std::string key = cache_key(pr, o);
    auto it = h->cache.find(key);
    if (it != h->cache.end()) {
        out = it->second;
        return DG_OK;
    }
    PlanResult r = plan_problem(pr, h->desc, o, h->eff.empty() ? nullptr : &h->eff);
    if (r.status != DG_OK) return fail(r.status, r.message);
    out = r.pareto.front();
    add_tail(pr, h->desc, out);
    h->cache.emplace(key, out);
    return DG_OK;
}

// ------------------------------------------------------- device description
// A small JSON reader for the probe's description (objects, strings, numbers,
// arrays, true/false/null).  Scalars come back flattened, the keys of nested
// objects joined with '.'; array contents are skipped.
struct JsonFlat {
    std::map<std::string, double> num;
    std::map<std::string, std::string> str;
};

class JsonReader {
  public:
    explicit JsonReader(const std::string &t) : t_(t) {}
    bool parse(JsonFlat &f)
    {
        ws();
        if (i_ >= t_.size() || t_[i_] != '{') return false;
        if (!value("", f, 0)) return false;
        ws();
        return i_ == t_.size();
    }

  private:
    const std::string &t_;
    size_t i_ = 0;
    void ws()
    {
        while (i_ < t_.size() && std::isspace((unsigned char)t_[i_])) ++i_;
    }
    bool lit(const char *w)
    {
        const size_t n = std::strlen(w);
        if (t_.compare(i_, n, w) != 0) return false;
        i_ += n;
        return true;
    }
    bool str(std::string &out)
    {
        if (i_ >= t_.size() || t_[i_] != '"') return false;
        ++i_;
        out.clear();
        while (i_ < t_.size() && t_[i_] != '"') {
            char c = t_[i_++];
            if (c == '\\') {
                if (i_ >= t_.size()) return false;
                const char e = t_[i_++];
                if (e == 'u') {
                    if (i_ + 4 > t_.size()) return false;
                    i_ += 4;
                    c = '?';
                } else {
                    c = e == 'n' ? '\n' : e == 't' ? '\t' : e == 'r' ? '\r' : e == 'b' ? '\b' : e == 'f' ? '\f' : e;
                }
            }
            out.push_back(c);
        }
        if (i_ >= t_.size()) return false;
        ++i_;
        return true;
    }
    bool value(const std::string &key, JsonFlat &f, int depth)
    {
        if (depth > 32) return false;
        ws();
        if (i_ >= t_.size()) return false;
        const char c = t_[i_];
        if (c == '{' || c == '[') {
            const bool obj = c == '{';
            const char close = obj ? '}' : ']';
            ++i_;
            ws();
            if (i_ < t_.size() && t_[i_] == close) {
                ++i_;
                return true;
            }
            JsonFlat skip;
            for (;;) {
                ws();
                std::string k;
                if (obj) {
                    if (!str(k)) return false;
                    ws();
                    if (i_ >= t_.size() || t_[i_] != ':') return false;
                    ++i_;
                }
                if (!value(obj ? (key.empty() ? k : key + "." + k) : "", obj ? f : skip, depth + 1)) return false;
                ws();
                if (i_ < t_.size() && t_[i_] == ',') {
                    ++i_;
                    continue;
                }
                if (i_ < t_.size() && t_[i_] == close) {
                    ++i_;
                    return true;
                }
                return false;
            }
        }
        if (c == '"') {
            std::string v;
            if (!str(v)) return false;
            f.str[key] = v;
            return true;
        }
        if (c == 't') return lit("true");
        if (c == 'f') return lit("false");
        if (c == 'n') return lit("null");
        const char *b = t_.c_str() + i_;
        char *e = nullptr;
        const double v = std::strtod(b, &e);
        if (e == b) return false;
        i_ += (size_t)(e - b);
        f.num[key] = v;
        return true;
    }
};

bool desc_fields_valid(const dg_device_desc &d)
{
    return d.cu_count > 0 && d.simd_per_cu > 0 && d.lds_bytes_per_cu > 0 && d.lds_bytes_per_wg > 0 &&
           d.vgpr_per_lane > 0 && d.max_waves_per_simd > 0 && d.clock_ghz > 0 && d.hbm_gbps > 0 &&
           d.l2_bytes_per_xcd >= 0 && d.mall_bytes >= 0 && d.mfma_tflops_f16 >= 0 && d.launch_us >= 0 &&
           d.lds_conflict_stride_words >= 0;
}

// Read the probe's JSON description into the handle (strict: every problem is
// an error; the caller decides whether to report it).
dg_status load_device_json(dg_handle_t h, const std::string &path)
{
    std::ifstream in(path);
    if (!in) return fail(DG_ERR_INVALID_ARG, "cannot read " + path);
    std::stringstream ss;
    ss << in.rdbuf();
    const std::string text = ss.str();
    JsonFlat f;
    if (!JsonReader(text).parse(f)) return fail(DG_ERR_INVALID_ARG, path + " is not a JSON object");
    dg_device_desc d = h->desc;
    const auto arch = f.str.find("arch");
    if (arch == f.str.end()) return fail(DG_ERR_INVALID_ARG, path + " names no arch");
    if (h->device >= 0 && arch->second != d.arch)
        return fail(DG_ERR_UNSUPPORTED, path + " describes " + arch->second + ", the device is " + d.arch);
    std::snprintf(d.arch, sizeof d.arch, "%s", arch->second.c_str());
    auto num = [&](const std::string &k, double &v) {
        const auto it = f.num.find(k);
        if (it == f.num.end()) return false;
        v = it->second;
        return true;
    };
    struct IntField {
        const char *name;
        int32_t *p;
    } ints[] = {{"cu_count", &d.cu_count}, {"xcd_count", &d.xcd_count}, {"simd_per_cu", &d.simd_per_cu},
                {"wave_size", &d.wave_size}, {"lds_bytes_per_cu", &d.lds_bytes_per_cu},
                {"lds_bytes_per_wg", &d.lds_bytes_per_wg}, {"vgpr_per_lane", &d.vgpr_per_lane},
                {"max_waves_per_simd", &d.max_waves_per_simd},
                {"lds_conflict_stride_words", &d.lds_conflict_stride_words}};
    struct DblField {
        const char *name;
        double *p;
    } dbls[] = {{"clock_ghz", &d.clock_ghz}, {"hbm_gbps", &d.hbm_gbps}, {"l2_bytes_per_xcd", &d.l2_bytes_per_xcd},
                {"mall_bytes", &d.mall_bytes}, {"mfma_tflops_f16", &d.mfma_tflops_f16}, {"launch_us", &d.launch_us}};
    // "desc" first, then "measured" (the probe's rates win)
    for (const char *sec : {"desc.", "measured."}) {
        for (auto &x : ints) {
            double v;
            if (num(std::string(sec) + x.name, v)) {
                if (v != std::floor(v) || std::fabs(v) > 1e9)
                    return fail(DG_ERR_INVALID_ARG, std::string(path) + ": " + sec + x.name + " is not an integer");
                *x.p = (int32_t)v;
            }
        }
        for (auto &x : dbls) {
            double v;
            if (num(std::string(sec) + x.name, v)) *x.p = v;
        }
    }
    if (!desc_fields_valid(d)) return fail(DG_ERR_INVALID_ARG, path + ": a field is out of range");
    if (h->device >= 0 && d.cu_count != h->desc.cu_count)
        return fail(DG_ERR_UNSUPPORTED, path + " describes " + std::to_string(d.cu_count) + " CUs, the device has " +
                                            std::to_string(h->desc.cu_count));
    EffTable eff;
    const std::string pre = "tiled_efficiency.", pre_r = "tiled_round_us.";
    for (const auto &kv : f.num) {
        if (kv.first.compare(0, pre.size(), pre) == 0) {
            if (!(kv.second > 0 && kv.second <= 1.5))
                return fail(DG_ERR_INVALID_ARG,
                            path + ": efficiency of " + kv.first.substr(pre.size()) + " out of (0, 1.5]");
            eff.eff[kv.first.substr(pre.size())] = kv.second;
        } else if (kv.first.compare(0, pre_r.size(), pre_r) == 0) {
            if (!(kv.second >= 0 && kv.second < 1e6))
                return fail(DG_ERR_INVALID_ARG,
                            path + ": round time of " + kv.first.substr(pre_r.size()) + " out of [0, 1e6) us");
            eff.round_us[kv.first.substr(pre_r.size())] = kv.second;
        }
    }
    d.calibrated = (int32_t)eff.size();
    h->desc = d;
    h->eff = std::move(eff);
    h->cache.clear();
    return DG_OK;
}

// <directory of this library>/devices/<arch>.json, or DG_DEVICE_JSON when set.
std::string default_device_json(const char *arch)
{
    if (const char *e = std::getenv("DG_DEVICE_JSON")) return e;
    Dl_info info;
    if (!dladdr(reinterpret_cast<void *>(&default_device_json), &info) || !info.dli_fname) return "";
    std::string dir = info.dli_fname;
    const size_t slash = dir.rfind('/');
    dir = slash == std::string::npos ? "." : dir.substr(0, slash);
    return dir + "/devices/" + arch + ".json";
}

const char *status_names[] = {"DG_OK",
                              "DG_ERR_INVALID_ARG",
                              "DG_ERR_UNSUPPORTED",
                              "DG_ERR_ALIGNMENT",
                              "DG_ERR_NO_CANDIDATE",
                              "DG_ERR_CONFLICT",
                              "DG_ERR_INVALID_STATE",
                              "DG_ERR_WORKSPACE",
                              "DG_ERR_HIP",
                              "DG_ERR_INTERNAL"};

}  // namespace

extern "C" {

dg_status dg_default_device_desc(dg_device_desc *out)
{
    if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
    std::memset(out, 0, sizeof *out);
    std::snprintf(out->arch, sizeof out->arch, "gfx950");
    out->cu_count = 256;
    out->xcd_count = 8;
    out->simd_per_cu = 4;
    out->wave_size = 64;
    out->lds_bytes_per_cu = 163840;
    out->lds_bytes_per_wg = 163840;
    out->vgpr_per_lane = 512;
    out->max_waves_per_simd = 8;
    out->clock_ghz = 2.4;
    out->hbm_gbps = 8000.0;
    out->l2_bytes_per_xcd = 4.0 * 1024 * 1024;
    out->mall_bytes = 256.0 * 1024 * 1024;
    // measured fields: unknown until probed (mfma_tflops_f16, launch_us,
    // lds_conflict_stride_words, calibrated = 0)
    return DG_OK;
}

dg_status dg_create(dg_handle_t *out, int hip_device)
{
    try {
        if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
        *out = nullptr;
        int n = 0;
        hipError_t e = hipGetDeviceCount(&n);
        if (e != hipSuccess || n <= 0) return fail(DG_ERR_HIP, "no HIP device visible");
        if (hip_device < 0 || hip_device >= n) return fail(DG_ERR_INVALID_ARG, "device index out of range");
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, hip_device);
        if (e != hipSuccess) return fail(DG_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return fail(DG_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", kernels are built for gfx950");
        // the static scratch of dg_gemm_noalloc: its address on this device
        e = scratch_init(hip_device);
        if (e != hipSuccess)
            return fail(DG_ERR_HIP, std::string("static scratch address: ") + hipGetErrorString(e));
        dg_handle_s *h = new dg_handle_s();
        dg_default_device_desc(&h->desc);
        h->desc.cu_count = prop.multiProcessorCount;
        if (prop.clockRate > 0) h->desc.clock_ghz = prop.clockRate / 1e6;
        if (prop.maxSharedMemoryPerMultiProcessor > 0)
            h->desc.lds_bytes_per_cu = (int32_t)prop.maxSharedMemoryPerMultiProcessor;
        h->device = hip_device;
        // the hardware probe's description of this device, when present
        const std::string json = default_device_json(h->desc.arch);
        if (!json.empty() && std::ifstream(json).good()) {
            const std::string saved = g_err;
            if (load_device_json(h, json) != DG_OK) g_err = saved;   // another device's: planned without it
        }
        {
            std::lock_guard<std::mutex> lk(g_live_mu);
            g_live.insert(h);
        }
        *out = h;
        return DG_OK;
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_create");
    }
}

dg_status dg_create_offline(dg_handle_t *out, const dg_device_desc *desc)
{
    try {
        if (!out || !desc) return fail(DG_ERR_INVALID_ARG, "NULL argument");
        *out = nullptr;
        if (!desc_fields_valid(*desc))
            return fail(DG_ERR_INVALID_ARG, "device description has a non-positive (or negative measured) field");
        dg_handle_s *h = new dg_handle_s();
        h->desc = *desc;
        h->desc.calibrated = 0;
        h->device = -1;
        {
            std::lock_guard<std::mutex> lk(g_live_mu);
            g_live.insert(h);
        }
        *out = h;
        return DG_OK;
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_create_offline");
    }
}

dg_status dg_destroy(dg_handle_t h)
{
    if (!h) return DG_OK;
    {
        std::lock_guard<std::mutex> lk(g_live_mu);
        if (!g_live.erase(h)) return fail(DG_ERR_INVALID_STATE, "handle is not live");
    }
    delete h;
    return DG_OK;
}

namespace {
bool desc_valid(const dg_device_desc *d) { return d && desc_fields_valid(*d); }
}  // namespace

dg_status dg_set_device_desc(dg_handle_t h, const dg_device_desc *desc)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (!desc_valid(desc)) return fail(DG_ERR_INVALID_ARG, "device description is NULL or has a non-positive field");
        h->desc = *desc;
        h->desc.calibrated = (int32_t)h->eff.size();
        h->cache.clear();
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_set_device_desc");
    }
}

dg_status dg_load_device_json(dg_handle_t h, const char *path)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (!path) return fail(DG_ERR_INVALID_ARG, "path is NULL");
        return load_device_json(h, path);
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_load_device_json");
    }
}

dg_status dg_get_device_desc(dg_handle_t h, dg_device_desc *out)
{
    if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
    if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
    *out = h->desc;
    return DG_OK;
}

dg_status dg_probe(dg_handle_t h, int32_t kind, const void *buf, size_t bytes, int32_t param, void *out,
                   int32_t grid, dg_stream_t stream)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: nothing is launched");
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
            return fail(DG_ERR_INVALID_STATE, "the current HIP device is not the handle's device");
        if (!out) return fail(DG_ERR_INVALID_ARG, "out is NULL");
        if (kind == DG_PROBE_STREAM) {
            if (!buf || bytes == 0 || bytes % 16 || grid <= 0 || param < 0 || (param >> 1) > 4096)
                return fail(DG_ERR_INVALID_ARG,
                            "stream probe: buf, a multiple of 16 bytes, grid > 0, 0 <= param, at most 4096 passes");
        } else if (kind == DG_PROBE_MFMA) {
            if (param < 0 || grid <= 0) return fail(DG_ERR_INVALID_ARG, "MFMA probe: param >= 0 and grid > 0");
        } else if (kind == DG_PROBE_LDS) {
            if (param < 1 || param > 16384) return fail(DG_ERR_INVALID_ARG, "LDS probe: 1 <= param <= 16384");
        } else if (kind == DG_PROBE_MFMA_DATA) {
            if (!buf || bytes < 16 || bytes % 16 || grid <= 0 || (param & 7) > 5 || (param >> 3) < 1)
                return fail(DG_ERR_INVALID_ARG,
                            "MFMA data probe: buf, a multiple of 16 bytes, grid > 0, mode 0..5, rounds >= 1");
        } else {
            return fail(DG_ERR_INVALID_ARG, "unknown probe kind");
        }
        const hipError_t he = launch_probe(kind, const_cast<void *>(buf), bytes, param, out, grid,
                                           reinterpret_cast<hipStream_t>(stream));
        if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("probe launch: ") + hipGetErrorString(he));
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_probe");
    }
}

dg_status dg_set_stage_clock(dg_handle_t h, uint64_t *buf, int64_t entries)
{
    if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
    if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: nothing is launched");
    if (entries < 0 || (!buf && entries > 0)) return fail(DG_ERR_INVALID_ARG, "stage clock: bad buffer size");
    h->clk = buf;
    h->clk_entries = buf ? entries : 0;
    return ok();
}

dg_status dg_plan(dg_handle_t h, int64_t M, int64_t N, int64_t K, const dg_dtypes *dt, const dg_layouts *lay,
                  int32_t group_k, int32_t epi_kind, const dg_plan_opts *opts, dg_plan_info *out)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        Problem pr;
        dg_status s = describe(M, N, K, dt, lay, group_k, epi_kind, 0, opts_or_default(opts).pad_k, pr);
        if (s) return s;
        Candidate c;
        s = plan_cached(h, pr, opts_or_default(opts), c);
        if (s) return s;
        if (out) fill_info(c, out);
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_plan");
    }
}

dg_status dg_plan_range(dg_handle_t h, int64_t M, int64_t N, int64_t K_min, int64_t K_max, const dg_dtypes *dt,
                        const dg_layouts *lay, int32_t group_k, int32_t epi_kind, const dg_plan_opts *opts,
                        dg_plan_opts *range_opts, dg_plan_info *out, double *worst_ratio)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (!range_opts) return fail(DG_ERR_INVALID_ARG, "range_opts is NULL");
        if (K_min < 0 || K_max < K_min) return fail(DG_ERR_INVALID_ARG, "K range must satisfy 0 <= K_min <= K_max");
        const dg_plan_opts o = opts_or_default(opts);
        if (o.force_m_tile || o.force_n_tile || o.force_k_tile || o.force_waves || o.force_mfma || o.force_path)
            return fail(DG_ERR_CONFLICT, "a K range plan chooses the variant: leave tile, K step, waves, MFMA block and path free");
        // every K of the range must be a valid problem; both ends decide that
        // (alignment and leading dimensions only tighten as K grows or shrinks)
        Problem lo, hi;
        dg_status s = describe(M, N, K_min, dt, lay, group_k, epi_kind, 0, o.pad_k, lo);
        if (s) return s;
        s = describe(M, N, K_max, dt, lay, group_k, epi_kind, 0, o.pad_k, hi);
        if (s) return s;
        // K samples: both ends and the doublings between them, on the MFMA depth
        // (any K with pad_k)
        const int64_t unit = o.pad_k ? 1 : (hi.path == P_MX ? 64 : ((hi.path == P_I8 || hi.path == P_E2M1) ? 32 : 16));
        std::vector<int64_t> ks{K_min};
        for (int64_t k = std::max<int64_t>(unit, K_min) * 2; k < K_max; k *= 2) ks.push_back(k / unit * unit);
        if (K_max != K_min) ks.push_back(K_max);
        std::vector<double> best(ks.size());
        for (size_t i = 0; i < ks.size(); ++i) {
            Problem pr;
            s = describe(M, N, ks[i], dt, lay, group_k, epi_kind, 0, o.pad_k, pr);
            if (s) return s;
            PlanResult r = plan_problem(pr, h->desc, o, h->eff.empty() ? nullptr : &h->eff);
            if (r.status != DG_OK) return fail(r.status, r.message);
            best[i] = r.pareto.front().est_us;
        }
        // candidate variants: each compiled tiled shape of the path, and the
        // streaming path with its split left to the planner
        struct Var {
            dg_plan_opts opt;
            double worst;
            int lds, regs;
        };
        std::vector<Var> vars;
        const TiledShape shapes[] = {
#define DG_TS(path, kmaj, bm, bn, wm, wn, kr, ms) {path, kmaj, bm, bn, wm, wn, kr, ms},
            DG_TILED_CATALOGUE(DG_TS)
#undef DG_TS
        };
        std::vector<dg_plan_opts> tries;
        for (const TiledShape &t : shapes) {
            if (t.path != hi.path || t.b_kmajor != hi.b_kmajor) continue;
            dg_plan_opts v = o;
            v.force_path = DG_PATH_TILED;
            v.force_m_tile = t.bm;
            v.force_n_tile = t.bn;
            v.force_waves = t.wm * t.wn;
            v.force_mfma = t.ms;
            v.force_k_tile = tiled_bk_elems(t.path) * t.kr;
            tries.push_back(v);
        }
        {
            dg_plan_opts v = o;
            v.force_path = DG_PATH_SKINNY;
            tries.push_back(v);
        }
        for (const dg_plan_opts &v : tries) {
            double worst = 0;
            int lds = 0, regs = 0;
            bool ok = true;
            for (size_t i = 0; i < ks.size() && ok; ++i) {
                Problem pr;
                s = describe(M, N, ks[i], dt, lay, group_k, epi_kind, 0, o.pad_k, pr);
                if (s) return s;   // (every sample passed above; kept for safety)
                PlanResult r = plan_problem(pr, h->desc, v, h->eff.empty() ? nullptr : &h->eff);
                if (r.status != DG_OK) {
                    ok = false;
                    break;
                }
                worst = std::max(worst, r.pareto.front().est_us / std::max(best[i], 1e-9));
                lds = std::max(lds, r.pareto.front().lds);
                regs = std::max(regs, r.pareto.front().vgpr + r.pareto.front().agpr);
            }
            if (ok) vars.push_back(Var{v, worst, lds, regs});
        }
        if (vars.empty()) return fail(DG_ERR_NO_CANDIDATE, "No valid candidate found after pruning for every K of the range");
        // the smallest worst-case ratio to the best plan of each K; then fewer
        // LDS bytes; then fewer registers; then catalogue order (deterministic)
        size_t bi = 0;
        for (size_t i = 1; i < vars.size(); ++i) {
            const Var &a = vars[i], &b = vars[bi];
            const bool tie = std::abs(a.worst - b.worst) <= 1e-12;
            if (a.worst < b.worst - 1e-12 || (tie && a.lds < b.lds) || (tie && a.lds == b.lds && a.regs < b.regs))
                bi = i;
        }
        *range_opts = vars[bi].opt;
        if (worst_ratio) *worst_ratio = vars[bi].worst;
        if (out) {
            Candidate c;
            s = plan_cached(h, hi, vars[bi].opt, c);
            if (s) return s;
            fill_info(c, out);
        }
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_plan_range");
    }
}

dg_status dg_plan_candidates(dg_handle_t h, int64_t M, int64_t N, int64_t K, const dg_dtypes *dt,
                             const dg_layouts *lay, int32_t group_k, int32_t epi_kind,
                             const dg_plan_opts *opts, dg_plan_info *out, int32_t cap, int32_t *count)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (cap < 0 || (cap > 0 && !out)) return fail(DG_ERR_INVALID_ARG, "bad output array");
        dg_plan_opts o = opts_or_default(opts);
        if (o.pad_k < 0 || o.pad_k > 1) return fail(DG_ERR_INVALID_ARG, "pad_k is 0 or 1");
        Problem pr;
        dg_status s = describe(M, N, K, dt, lay, group_k, epi_kind, 0, o.pad_k, pr);
        if (s) return s;
        PlanResult r = plan_problem(pr, h->desc, o, h->eff.empty() ? nullptr : &h->eff);
        if (r.status != DG_OK) return fail(r.status, r.message);
        if (count) *count = (int32_t)r.pareto.size();
        for (int i = 0; i < cap && i < (int)r.pareto.size(); ++i) {
            add_tail(pr, h->desc, r.pareto[i]);
            fill_info(r.pareto[i], &out[i]);
        }
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_plan_candidates");
    }
}

}  // extern "C"

namespace {

// dg_gemm and dg_gemm_noalloc.  ws_limit >= 0: the workspace is the static
// scratch of that many bytes, and the planner only keeps plans that fit it.
dg_status gemm_impl(dg_handle_t h, int64_t M, int64_t N, int64_t K, const dg_dtypes *dt, const dg_layouts *lay,
                    const void *A, const void *B, const void *b_scale, int32_t group_k, const void *D, void *C,
                    const void *alpha, const void *beta, const dg_epilogue *epi, const dg_plan_opts *opts,
                    void *workspace, size_t workspace_bytes, dg_stream_t stream, int64_t ws_limit)
{
    {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: planning only");
        if (!dt || !alpha || !beta) return fail(DG_ERR_INVALID_ARG, "dtypes, alpha and beta are required");
        if (dt->a == DG_F8E4M3)
            return fail(DG_ERR_UNSUPPORTED, "MX operands carry scales for A: call dg_gemm_mx");
        const bool is_int = dt->compute == DG_I32;
        const int32_t ia = is_int ? *reinterpret_cast<const int32_t *>(alpha) : 0;
        const int32_t ib = is_int ? *reinterpret_cast<const int32_t *>(beta) : 0;
        const float fa = is_int ? 0.f : *reinterpret_cast<const float *>(alpha);
        const float fb = is_int ? 0.f : *reinterpret_cast<const float *>(beta);
        const int beta_nz = is_int ? ib != 0 : fb != 0.f;
        dg_epilogue E{};
        if (epi) E = *epi;
        Problem pr;
        dg_status s = describe(M, N, K, dt, lay, group_k, E.kind, beta_nz, opts_or_default(opts).pad_k, pr);
        if (s) return s;
        pr.ws_limit = ws_limit;
        const bool rq = E.kind == DG_EPI_REQUANT_I8 || E.kind == DG_EPI_REQUANT_F16;
        if (rq && ia != 1) return fail(DG_ERR_INVALID_ARG, "requantise epilogues need alpha == 1 (use epi->scale)");
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
            return fail(DG_ERR_INVALID_STATE, "the current HIP device is not the handle's device");
        if (M == 0 || N == 0) return ok();
        // operands
        if (!C) return fail(DG_ERR_INVALID_ARG, "C is NULL");
        if (K > 0 && (!A || !B)) return fail(DG_ERR_INVALID_ARG, "A or B is NULL");
        if (pr.path == P_E2M1 && K > 0 && !b_scale) return fail(DG_ERR_INVALID_ARG, "e2m1 needs b_scale");
        if (beta_nz && !D) return fail(DG_ERR_INVALID_ARG, "beta != 0 needs D");
        const bool has_bias_kind = E.kind == DG_EPI_BIAS || E.kind == DG_EPI_BIAS_GELU_ERF;
        if (has_bias_kind && !E.bias) return fail(DG_ERR_INVALID_ARG, "the epilogue needs a bias");
        if (E.bias) {
            if (rq && E.bias_type != DG_F32) return fail(DG_ERR_UNSUPPORTED, "requantise bias must be F32");
            if (!rq && E.bias_type != DG_F16 && E.bias_type != DG_BF16 && E.bias_type != DG_F32)
                return fail(DG_ERR_UNSUPPORTED, "bias must be F16, BF16 or F32");
            if (!rq && E.kind != DG_EPI_BIAS && E.kind != DG_EPI_BIAS_GELU_ERF)
                return fail(DG_ERR_CONFLICT, "a bias was given to an epilogue without a bias term");
        }
        if ((A && !aligned(A, 16)) || (B && !aligned(B, 16)))
            return fail(DG_ERR_ALIGNMENT, "A and B must be 16-byte aligned");
        const int osz = elt_size(pr.out_type);
        if (!aligned(C, osz) || (D && !aligned(D, osz)) || (b_scale && !aligned(b_scale, 4)))
            return fail(DG_ERR_ALIGNMENT, "C or D is misaligned for its type, or b_scale is not 4-byte aligned");
        dg_layouts L{};
        if (lay) L = *lay;
        // plan
        const dg_plan_opts o = opts_or_default(opts);
        Candidate c;
        s = plan_cached(h, pr, o, c);
        if (s) return s;
        if (c.family == F_TILED) {
            const int64_t la = L.lda ? L.lda : K, lb = L.ldb ? L.ldb : (pr.b_kmajor ? K : N);
            const int64_t ea = (pr.path == P_I8 || pr.path == P_MX) ? 1 : 2;
            const int64_t eb = pr.path == P_E2M1 ? 1 : ea;   // e2m1: ldb counts codes, 2 per byte
            const int64_t b_ext = pr.b_kmajor ? N * lb * eb / (pr.path == P_E2M1 ? 2 : 1) : K * lb * eb;
            if (M * la * ea >= (int64_t(1) << 32) || b_ext >= (int64_t(1) << 32) ||
                (pr.path == P_E2M1 && (K / 32) * (N + (N & 1)) * 2 >= (int64_t(1) << 32)))
                return fail(DG_ERR_UNSUPPORTED, "an operand spans 4 GiB or more (32-bit offsets of the tiled path)");
        }
        if (ws_limit >= 0 && c.ws_bytes > ws_limit)
            return fail(DG_ERR_WORKSPACE, "the plan's partial sums need " + std::to_string(c.ws_bytes) +
                                              " bytes; the static scratch holds " + std::to_string(ws_limit));
        if (c.ws_bytes > 0 && (!workspace || workspace_bytes < (size_t)c.ws_bytes))
            return fail(DG_ERR_WORKSPACE, "workspace missing or smaller than " + std::to_string(c.ws_bytes) + " bytes");
        if (c.ws_bytes > 0 && !aligned(workspace, 16)) return fail(DG_ERR_ALIGNMENT, "workspace must be 16-byte aligned");

        EpiArgs ea{};
        ea.C = C;
        ea.D = D;
        ea.bias = E.bias;
        ea.ldc = L.ldc ? L.ldc : N;
        ea.ldd = L.ldd ? L.ldd : N;
        ea.alpha = fa;
        ea.beta = fb;
        ea.ialpha = ia;
        ea.ibeta = ib;
        ea.rq_scale = E.scale;
        ea.kind = E.kind;
        ea.out_type = pr.out_type;
        ea.bias_type = elt_of(E.bias_type);
        ea.d_read = beta_nz;
        const int64_t lda = L.lda ? L.lda : K;
        const int64_t ldb = L.ldb ? L.ldb : (pr.b_kmajor ? K : N);
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        hipError_t he = hipSuccess;
        // pad_k: the planned kernels cover the aligned part of K (pr.K) and write
        // partials; a tail kernel adds the last k_pad elements as one more slice.
        const int s_main = c.split_k;   // 0 when pad_k leaves no aligned part
        const int s_all = s_main + (c.k_pad ? 1 : 0);
        const int s_arg = c.k_pad ? s_all : c.split_k;   // > 1: the kernels write partials
        if (s_main == 0) {
            // nothing but the tail: the aligned part of K is empty
        } else if (c.family == F_TILED) {
            TiledArgs ta{};
            ta.A = A;
            ta.B = B;
            ta.scale = b_scale;
            ta.lda = lda;
            ta.ldb = ldb;
            ta.ld_scale = N + (N & 1);   // e2m1 scales: group rows of N rounded up to even
            ta.M = (int)M;
            ta.N = (int)N;
            ta.K = (int)pr.K;
            ta.split_k = s_arg;
            ta.k_slice = c.k_slice;
            ta.tiles_m = (int)((M + c.m_tile - 1) / c.m_tile);
            ta.tiles_n = (int)((N + c.n_tile - 1) / c.n_tile);
            ta.group_m = 4;
            ta.ws = workspace;
            ta.epi = ea;
            ta.clk = reinterpret_cast<unsigned long long *>(h->clk);
            ta.clk_wgs = h->clk ? h->clk_entries / 8 : 0;
            he = launch_tiled(c.kernel_id, ta, c.grid_x, c.grid_y, st);
        } else {
            SkinnyArgs sa{};
            sa.A = A;
            sa.B = B;
            sa.scale = b_scale;
            sa.lda = lda;
            sa.ldb = ldb;
            sa.ld_scale = N + (N & 1);
            sa.M = (int)M;
            sa.N = (int)N;
            sa.K = (int)pr.K;
            sa.split_k = s_arg;
            sa.k_slice = c.k_slice;
            sa.ws = workspace;
            sa.epi = ea;
            if (c.family == F_SKINNY_VALU) he = launch_skinny_valu(c.kernel_id, sa, c.grid_x, c.grid_y, st);
            else if (c.family == F_SKINNY_MFMA) he = launch_skinny_mfma(c.kernel_id, sa, c.grid_x, c.grid_y, st);
            else he = launch_skinny_e2m1(c.kernel_id, sa, c.grid_x, c.grid_y, st);
        }
        if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(he));
        if (c.k_pad) {
            TailArgs tl{};
            tl.A = A;
            tl.B = B;
            tl.lda = lda;
            tl.ldb = ldb;
            tl.M = (int)M;
            tl.N = (int)N;
            tl.k0 = (int)pr.K;
            tl.k1 = (int)K;
            tl.path = pr.path;
            tl.b_kmajor = pr.b_kmajor;
            tl.ws = static_cast<char *>(workspace) + (int64_t)s_main * M * N * 4;
            he = launch_tail(tl, st);
            if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("tail launch: ") + hipGetErrorString(he));
        }
        if (s_all > 1 || c.k_pad) {
            ReduceArgs ra{};
            ra.ws = workspace;
            ra.split_k = s_all;
            ra.M = (int)M;
            ra.N = (int)N;
            ra.is_int = pr.path == P_I8;
            // runs per output: enough threads to keep loads in flight (about 64K),
            // at most 16 and at most the slices; few slices need no runs
            {
                const int64_t groups = std::max<int64_t>(1, M * N / 4);
                int runs = 1;
                while (runs < 16 && runs * 2 <= s_all && groups * runs < 65536) runs *= 2;
                ra.lanes = s_all <= 8 ? 1 : runs;
            }
            ra.epi = ea;
            he = launch_reduce(ra, st);
            if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("reduce launch: ") + hipGetErrorString(he));
        }
        return ok();
    }
}

}  // namespace

extern "C" {

dg_status dg_gemm(dg_handle_t h, int64_t M, int64_t N, int64_t K, const dg_dtypes *dt, const dg_layouts *lay,
                  const void *A, const void *B, const void *b_scale, int32_t group_k, const void *D, void *C,
                  const void *alpha, const void *beta, const dg_epilogue *epi, const dg_plan_opts *opts,
                  void *workspace, size_t workspace_bytes, dg_stream_t stream)
{
    try {
        return gemm_impl(h, M, N, K, dt, lay, A, B, b_scale, group_k, D, C, alpha, beta, epi, opts, workspace,
                         workspace_bytes, stream, -1);
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_gemm");
    }
}

dg_status dg_gemm_noalloc(dg_handle_t h, int64_t M, int64_t N, int64_t K, const dg_dtypes *dt,
                          const dg_layouts *lay, const void *A, const void *B, const void *b_scale,
                          int32_t group_k, const void *D, void *C, const void *alpha, const void *beta,
                          const dg_epilogue *epi, const dg_plan_opts *opts, dg_stream_t stream)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: planning only");
        // the address dg_create looked up on the handle's device (never the
        // array's host-side name)
        void *ptr = scratch_ptr(h->device);
        if (!ptr) return fail(DG_ERR_INVALID_STATE, "no static scratch address for the handle's device");
        return gemm_impl(h, M, N, K, dt, lay, A, B, b_scale, group_k, D, C, alpha, beta, epi, opts, ptr,
                         DG_SCRATCH_BYTES, stream, DG_SCRATCH_BYTES);
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_gemm_noalloc");
    }
}

dg_status dg_gemm_mx(dg_handle_t h, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     const void *a_scale, int64_t lda_scale, const void *B, int64_t ldb, const void *b_scale,
                     int64_t ldb_scale, void *C, int32_t c_type, int64_t ldc, float alpha,
                     const dg_epilogue *epi, const dg_plan_opts *opts, void *workspace, size_t workspace_bytes,
                     dg_stream_t stream)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: planning only");
        dg_epilogue E{};
        if (epi) E = *epi;
        if (E.kind == DG_EPI_REQUANT_I8 || E.kind == DG_EPI_REQUANT_F16)
            return fail(DG_ERR_UNSUPPORTED, "requantise epilogues need the int8 path");
        const dg_dtypes dt{DG_F8E4M3, DG_E2M1, c_type, DG_F32};
        const int64_t G = K / 32;
        const int64_t la = lda ? lda : K, lb = ldb ? ldb : K;
        const int64_t lsa = lda_scale ? lda_scale : (M + 3) / 4 * 4;   // group-major scale rows
        const int64_t lsb = ldb_scale ? ldb_scale : (N + 3) / 4 * 4;
        if (lda < 0 || ldb < 0 || lda_scale < 0 || ldb_scale < 0 || ldc < 0)
            return fail(DG_ERR_INVALID_ARG, "negative leading dimension");
        const dg_layouts L{DG_ROW_MAJOR, DG_COL_MAJOR, la, lb, ldc ? ldc : N, N};
        const dg_plan_opts o = opts_or_default(opts);
        if (o.pad_k) return fail(DG_ERR_UNSUPPORTED, "the MX path needs K in whole 64-element MFMA steps");
        Problem pr;
        dg_status s = describe(M, N, K, &dt, &L, 32, E.kind, 0, 0, pr);
        if (s) return s;
        if (K > 0 && (lsa < M || lsb < N))
            return fail(DG_ERR_INVALID_ARG, "a scale leading dimension is smaller than M (a_scale) or N (b_scale)");
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
            return fail(DG_ERR_INVALID_STATE, "the current HIP device is not the handle's device");
        if (M == 0 || N == 0) return ok();
        if (!C) return fail(DG_ERR_INVALID_ARG, "C is NULL");
        if (K > 0 && (!A || !B || !a_scale || !b_scale))
            return fail(DG_ERR_INVALID_ARG, "A, B and both scale arrays are required");
        const bool has_bias_kind = E.kind == DG_EPI_BIAS || E.kind == DG_EPI_BIAS_GELU_ERF;
        if (has_bias_kind && !E.bias) return fail(DG_ERR_INVALID_ARG, "the epilogue needs a bias");
        if (E.bias) {
            if (E.bias_type != DG_F16 && E.bias_type != DG_BF16 && E.bias_type != DG_F32)
                return fail(DG_ERR_UNSUPPORTED, "bias must be F16, BF16 or F32");
            if (!has_bias_kind) return fail(DG_ERR_CONFLICT, "a bias was given to an epilogue without a bias term");
        }
        if ((A && !aligned(A, 16)) || (B && !aligned(B, 16)))
            return fail(DG_ERR_ALIGNMENT, "A and B must be 16-byte aligned");
        if (K > 0 && (lsa % 4 || lsb % 4 || !aligned(a_scale, 4) || !aligned(b_scale, 4)))
            return fail(DG_ERR_ALIGNMENT, "scale arrays: 4-byte aligned pointers and leading dimensions");
        const int osz = elt_size(pr.out_type);
        if (!aligned(C, osz)) return fail(DG_ERR_ALIGNMENT, "C is misaligned for its type");
        Candidate c;
        s = plan_cached(h, pr, o, c);
        if (s) return s;
        if (c.family != F_TILED) return fail(DG_ERR_INTERNAL, "MX plan is not a tiled plan");
        if (M * la >= (int64_t(1) << 32) || N * lb / 2 >= (int64_t(1) << 32) || G * lsa >= (int64_t(1) << 32) ||
            G * lsb >= (int64_t(1) << 32))
            return fail(DG_ERR_UNSUPPORTED, "an operand spans 4 GiB or more (32-bit offsets of the tiled path)");
        if (c.ws_bytes > 0 && (!workspace || workspace_bytes < (size_t)c.ws_bytes))
            return fail(DG_ERR_WORKSPACE, "workspace missing or smaller than " + std::to_string(c.ws_bytes) + " bytes");
        if (c.ws_bytes > 0 && !aligned(workspace, 16)) return fail(DG_ERR_ALIGNMENT, "workspace must be 16-byte aligned");

        EpiArgs ea{};
        ea.C = C;
        ea.bias = E.bias;
        ea.ldc = L.ldc;
        ea.ldd = N;
        ea.alpha = alpha;
        ea.kind = E.kind;
        ea.out_type = pr.out_type;
        ea.bias_type = elt_of(E.bias_type);
        TiledArgs ta{};
        ta.A = A;
        ta.B = B;
        ta.scale = b_scale;
        ta.scale_a = a_scale;
        ta.lda = la;
        ta.ldb = lb;
        ta.ld_scale = lsb;
        ta.ld_scale_a = lsa;
        ta.M = (int)M;
        ta.N = (int)N;
        ta.K = (int)K;
        ta.split_k = c.split_k;
        ta.k_slice = c.k_slice;
        ta.tiles_m = (int)((M + c.m_tile - 1) / c.m_tile);
        ta.tiles_n = (int)((N + c.n_tile - 1) / c.n_tile);
        ta.group_m = 4;
        ta.ws = workspace;
        ta.epi = ea;
        ta.clk = reinterpret_cast<unsigned long long *>(h->clk);
        ta.clk_wgs = h->clk ? h->clk_entries / 8 : 0;
        hipStream_t st = reinterpret_cast<hipStream_t>(stream);
        hipError_t he = launch_tiled(c.kernel_id, ta, c.grid_x, c.grid_y, st);
        if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(he));
        if (c.split_k > 1) {
            ReduceArgs ra{};
            ra.ws = workspace;
            ra.split_k = c.split_k;
            ra.M = (int)M;
            ra.N = (int)N;
            ra.is_int = 0;
            const int64_t groups = std::max<int64_t>(1, M * N / 4);
            int runs = 1;
            while (runs < 16 && runs * 2 <= c.split_k && groups * runs < 65536) runs *= 2;
            ra.lanes = c.split_k <= 8 ? 1 : runs;
            ra.epi = ea;
            he = launch_reduce(ra, st);
            if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("reduce launch: ") + hipGetErrorString(he));
        }
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_gemm_mx");
    }
}

dg_status dg_quant_mx(dg_handle_t h, int64_t M, int64_t K, const void *X, int64_t ldx, void *codes, int64_t ldq,
                      void *scales, int64_t ld_scale, dg_stream_t stream)
{
    try {
        if (!is_live(h)) return fail(DG_ERR_INVALID_STATE, "handle is NULL or destroyed");
        if (h->device < 0) return fail(DG_ERR_INVALID_STATE, "offline handle: nothing is launched");
        if (M < 0 || K < 0 || ldx < 0 || ldq < 0 || ld_scale < 0)
            return fail(DG_ERR_INVALID_ARG, "negative size or leading dimension");
        if (M > INT32_MAX || K > INT32_MAX) return fail(DG_ERR_UNSUPPORTED, "sizes above 2^31-1 are not supported");
        if (K % 32) return fail(DG_ERR_ALIGNMENT, "K is not a multiple of the 32-value scale block");
        const int64_t lx = ldx ? ldx : K, lq = ldq ? ldq : K, ls = ld_scale ? ld_scale : M;
        if (lx < K || lq < K || ls < M) return fail(DG_ERR_INVALID_ARG, "a leading dimension is smaller than the matrix");
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess || cur != h->device)
            return fail(DG_ERR_INVALID_STATE, "the current HIP device is not the handle's device");
        if (M == 0 || K == 0) return ok();
        if (!X || !codes || !scales) return fail(DG_ERR_INVALID_ARG, "X, codes and scales are required");
        if (!aligned(X, 16) || !aligned(codes, 16) || (lx * 2) % 16 || lq % 16)
            return fail(DG_ERR_ALIGNMENT, "X and codes: 16-byte aligned pointers and rows");
        QuantMxArgs qa{};
        qa.X = X;
        qa.codes = codes;
        qa.scales = scales;
        qa.ldx = lx;
        qa.ldq = lq;
        qa.ld_scale = ls;
        qa.M = (int)M;
        qa.K = (int)K;
        const hipError_t he = launch_quant_mx(qa, reinterpret_cast<hipStream_t>(stream));
        if (he != hipSuccess) return fail(DG_ERR_HIP, std::string("quantiser launch: ") + hipGetErrorString(he));
        return ok();
    } catch (...) {
        return fail(DG_ERR_INTERNAL, "exception in dg_quant_mx");
    }
}

const char *dg_last_error(void) { return g_err.c_str(); }

const char *dg_status_str(dg_status s)
{
    if ((int)s < 0 || (int)s >= (int)(sizeof(status_names) / sizeof(status_names[0]))) return "DG_UNKNOWN";
    return status_names[s];
}

}  // extern "C"
