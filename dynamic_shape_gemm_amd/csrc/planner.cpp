// Run-time polymerizer (see planner.h for the model and its sources).
#include "planner.h"

#include <algorithm>
#include <array>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <limits>
#include <sstream>
#include <numeric>
#include <unordered_map>

namespace mkp {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Exact division by a fixed positive divisor through its reciprocal: a 64-bit
// integer division costs tens of cycles and the search divides a few times
// per candidate.  For 0 <= x < 2^50 the product x * (1/d) is within 0.25 of
// x / d, so one correction step makes the quotient exact; larger x divide.
struct FastDiv {
    int64_t d = 1;
    double inv = 1.0;
    void set(int64_t v) {
        d = v;
        inv = 1.0 / (double)v;
    }
    int64_t quot(int64_t x, int64_t& rem) const {
        if (x >= (int64_t(1) << 50)) {
            rem = x % d;
            return x / d;
        }
        int64_t q = (int64_t)((double)x * inv);
        int64_t r = x - q * d;
        if (r < 0) {
            --q;
            r += d;
        } else if (r >= d) {
            ++q;
            r -= d;
        }
        rem = r;
        return q;
    }
    int64_t ceil(int64_t x) const {
        int64_t r;
        const int64_t q = quot(x, r);
        return q + (r != 0);
    }
};

bool parse_table(const std::string& text, PerfTable& out, std::string& err) {
    PerfTable t;
    t.kernels.clear();
    std::istringstream in(text);
    std::string raw;
    int lineno = 0;
    struct CurveLine {
        int kind;   // 0 g, 1 tail, 2 tailx
        int rows;   // 0: square wave
        std::string name;
        std::vector<std::pair<double, double>> pts;
    };
    std::vector<CurveLine> curves;
    std::vector<std::pair<std::string, std::string>> pair_names;
    while (std::getline(in, raw)) {
        ++lineno;
        auto hash = raw.find('#');
        std::string line = hash == std::string::npos ? raw : raw.substr(0, hash);
        std::istringstream ls(line);
        std::string key;
        if (!(ls >> key)) continue;
        auto fail = [&](const std::string& what) {
            err = "table line " + std::to_string(lineno) + ": " + what;
            return false;
        };
        if (key == "device") {
            if (!(ls >> t.cus) || t.cus <= 0) return fail("bad device line");
        } else if (key == "launch_us") {
            if (!(ls >> t.launch_us) || t.launch_us < 0) return fail("bad launch_us");
        } else if (key == "reduce") {
            if (!(ls >> t.red_launch_us >> t.red_gbps) || t.red_gbps <= 0) return fail("bad reduce line");
        } else if (key == "transpose") {
            // transpose <launch_us> <GB/s>: K x N -> N x K copy of B
            if (!(ls >> t.tr_launch_us >> t.tr_gbps) || t.tr_gbps <= 0 || t.tr_launch_us < 0)
                return fail("bad transpose line");
        } else if (key == "splitk") {
            t.splits.clear();
            int s;
            while (ls >> s) {
                if (s < 1) return fail("split factor < 1");
                t.splits.push_back(s);
            }
            if (t.splits.empty()) return fail("empty splitk");
        } else if (key == "measured") {
            // measured <mfma_tflops> <copy_gbps> [<read_gbps>]: sustained
            // ceilings, reported only
            if (!(ls >> t.mfma_tflops >> t.hbm_gbps)) return fail("bad measured line");
            double rd = 0.0;
            if (ls >> rd) t.hbm_read_gbps = rd;
        } else if (key == "patterns") {
            t.pat_I = t.pat_IIM = t.pat_IIN = false;
            std::string p;
            while (ls >> p) {
                if (p == "I") t.pat_I = true;
                else if (p == "II-M") t.pat_IIM = true;
                else if (p == "II-N") t.pat_IIN = true;
                else return fail("unknown pattern");
            }
        } else if (key == "kernel") {
            TableKernel k;
            if (!(ls >> k.name >> k.uM >> k.uN >> k.uK >> k.wg_per_cu)) return fail("bad kernel line");
            std::string layout;   // optional: kn (B is K x N, the default) or nk
            if (ls >> layout) {
                if (layout == "nk") k.bt = true;
                else if (layout != "kn") return fail("kernel layout must be kn or nk");
            }
            if (k.uM <= 0 || k.uN <= 0 || k.uK <= 0 || k.wg_per_cu <= 0) return fail("bad kernel tile");
            for (auto& e : t.kernels)
                if (e.name == k.name) return fail("duplicate kernel");
            t.kernels.push_back(k);
        } else if (key == "rows") {
            // rows <r1> <r2> ...: tile-row classes with curves of their own
            int r;
            while (ls >> r) {
                if (r <= 0 || r > 4096 || (!t.row_classes.empty() && r <= t.row_classes.back()) || t.row_classes.size() >= 7)
                    return fail("rows must be at most 7 increasing counts in 1..4096");
                t.row_classes.push_back(r);
            }
        } else if (key.rfind("g", 0) == 0 || key.rfind("tail", 0) == 0) {
            // g[@r] <kernel> <t>:<us> ...           (full-wave time per K steps)
            // tail[x][@r] <kernel> <f>:<ratio> ...  (partial-wave time relative to a full wave)
            CurveLine cl;
            const auto at = key.find('@');
            const std::string base = key.substr(0, at);
            cl.kind = base == "g" ? 0 : base == "tail" ? 1 : base == "tailx" ? 2 : -1;
            if (cl.kind < 0) return fail("unknown key");
            cl.rows = 0;
            if (at != std::string::npos && ((cl.rows = std::atoi(key.c_str() + at + 1)) <= 0))
                return fail("bad row class in " + key);
            std::string tok;
            if (!(ls >> cl.name)) return fail("bad curve line");
            while (ls >> tok) {
                auto c = tok.find(':');
                if (c == std::string::npos) return fail("bad curve point");
                double x = std::atof(tok.substr(0, c).c_str());
                double y = std::atof(tok.substr(c + 1).c_str());
                if (cl.kind == 0 ? !(x > 0) || !(y >= 0) : !(x > 0 && x < 1) || !(y > 0 && y <= 1))
                    return fail(cl.kind == 0 ? "bad g value" : "bad tail value");
                cl.pts.emplace_back(x, y);
            }
            curves.push_back(std::move(cl));
        } else if (key == "pair") {
            // pair <kernel a> <kernel b>: a and b can share one launch
            std::string a, b;
            if (!(ls >> a >> b) || a == b) return fail("bad pair line");
            pair_names.emplace_back(a, b);
        } else {
            return fail("unknown key");
        }
    }
    for (auto& k : t.kernels) k.by_rows.assign(t.row_classes.size(), Curves{});
    for (auto& cl : curves) {
        int set = -1;   // -1: square
        if (cl.rows > 0) {
            for (size_t i = 0; i < t.row_classes.size(); ++i)
                if (t.row_classes[i] == cl.rows) set = (int)i;
            if (set < 0) {
                err = "curve for row class " + std::to_string(cl.rows) + " not listed in rows";
                return false;
            }
        }
        bool found = false;
        for (auto& k : t.kernels)
            if (k.name == cl.name) {
                auto& dst = set < 0 ? (cl.kind == 0 ? k.pts : cl.kind == 1 ? k.tail : k.tailx)
                                    : (cl.kind == 0 ? k.by_rows[set].pts : cl.kind == 1 ? k.by_rows[set].tail
                                                                                         : k.by_rows[set].tailx);
                dst.insert(dst.end(), cl.pts.begin(), cl.pts.end());
                found = true;
            }
        if (!found) {
            err = "curve line for unknown kernel " + cl.name;
            return false;
        }
    }
    for (auto& k : t.kernels) {
        for (auto* v : {&k.tail, &k.tailx, &k.pts}) std::sort(v->begin(), v->end());
        for (auto& c : k.by_rows)
            for (auto* v : {&c.tail, &c.tailx, &c.pts}) std::sort(v->begin(), v->end());
        if (k.pts.empty()) {
            err = "kernel " + k.name + " has no g points";
            return false;
        }
    }
    if (t.kernels.empty()) {
        err = "table has no kernels";
        return false;
    }
    for (auto& pn : pair_names) {
        int ia = -1, ib = -1;
        for (size_t i = 0; i < t.kernels.size(); ++i) {
            if (t.kernels[i].name == pn.first) ia = (int)i;
            if (t.kernels[i].name == pn.second) ib = (int)i;
        }
        if (ia < 0 || ib < 0) {
            err = "pair line names an unknown kernel: " + pn.first + " " + pn.second;
            return false;
        }
        if (t.kernels[ia].bt != t.kernels[ib].bt || t.kernels[ia].wg_per_cu != t.kernels[ib].wg_per_cu) {
            err = "pair " + pn.first + " " + pn.second + " differs in B layout or workgroups per CU";
            return false;
        }
        t.pairs.emplace_back(ia, ib);
    }
    out = t;
    return true;
}

std::string table_to_text(const PerfTable& t) {
    std::ostringstream o;
    o.precision(9);
    o << "device " << t.cus << "\n";
    o << "launch_us " << t.launch_us << "\n";
    o << "reduce " << t.red_launch_us << " " << t.red_gbps << "\n";
    if (t.tr_gbps > 0) o << "transpose " << t.tr_launch_us << " " << t.tr_gbps << "\n";
    o << "splitk";
    for (int s : t.splits) o << " " << s;
    o << "\npatterns" << (t.pat_I ? " I" : "") << (t.pat_IIM ? " II-M" : "") << (t.pat_IIN ? " II-N" : "")
      << "\n";
    if (t.mfma_tflops > 0 || t.hbm_gbps > 0) {
        o << "measured " << t.mfma_tflops << " " << t.hbm_gbps;
        if (t.hbm_read_gbps > 0) o << " " << t.hbm_read_gbps;
        o << "\n";
    }
    for (auto& k : t.kernels)
        o << "kernel " << k.name << " " << k.uM << " " << k.uN << " " << k.uK << " " << k.wg_per_cu
          << (k.bt ? " nk" : "") << "\n";
    if (!t.row_classes.empty()) {
        o << "rows";
        for (int r : t.row_classes) o << " " << r;
        o << "\n";
    }
    static const char* const kCurve[] = {"g", "tail", "tailx"};
    for (int set = -1; set < (int)t.row_classes.size(); ++set)
        for (int kind = 0; kind < 3; ++kind)
            for (auto& k : t.kernels) {
                const Curves* c = set >= 0 && set < (int)k.by_rows.size() ? &k.by_rows[set] : nullptr;
                if (set >= 0 && !c) continue;
                const auto& pts = kind == 0 ? (c ? c->pts : k.pts) : kind == 1 ? (c ? c->tail : k.tail)
                                                                                : (c ? c->tailx : k.tailx);
                if (pts.empty()) continue;
                o << kCurve[kind];
                if (set >= 0) o << "@" << t.row_classes[set];
                o << " " << k.name;
                for (auto& p : pts) o << " " << p.first << ":" << p.second;
                o << "\n";
            }
    for (auto& pr : t.pairs) o << "pair " << t.kernels[pr.first].name << " " << t.kernels[pr.second].name << "\n";
    return o.str();
}

double merged_makespan(int64_t S, int64_t n1, double d1, int64_t n2, double d2) {
    if (n1 <= 0) return (double)((n2 + S - 1) / S) * d2;
    const int64_t w1 = n1 / S, r1 = n1 % S;
    const double t0 = (double)w1 * d1;
    if (n2 <= 0) return r1 ? t0 + d1 : t0;
    if (r1 == 0) return t0 + (double)((n2 + S - 1) / S) * d2;
    // after w1 full waves, a = S - r1 slots are free at t0 and the r1 slots
    // of the first region's last wave at t1 = t0 + d1; the second region's
    // tasks take them in order, so its last task starts at the n2-th
    // smallest value of {t0 + i d2 (a of each)} u {t1 + j d2 (b of each)}
    const int64_t a = S - r1, b = r1;
    const double t1 = t0 + d1;
    const double q = d1 / d2;   // (t1 - t0) / d2
    const double eps = 1e-9;
    // starts at or before t0 + i d2: a (i + 1) + b (floor(i - q) + 1)_+
    auto count_a = [&](int64_t i) {
        const double jb = std::floor((double)i - q + eps);
        return a * (i + 1) + (jb >= 0 ? b * ((int64_t)jb + 1) : 0);
    };
    // starts at or before t1 + j d2: b (j + 1) + a (floor(j + q) + 1)
    auto count_b = [&](int64_t j) { return b * (j + 1) + a * ((int64_t)std::floor((double)j + q + eps) + 1); };
    auto first = [&](auto&& cnt) {   // smallest index whose count reaches n2
        int64_t lo = 0, hi = (n2 + std::min(a, b) - 1) / std::min(a, b);
        while (lo < hi) {
            const int64_t mid = (lo + hi) / 2;
            if (cnt(mid) >= n2) hi = mid;
            else lo = mid + 1;
        }
        return lo;
    };
    const double start = std::min(t0 + (double)first(count_a) * d2, t1 + (double)first(count_b) * d2);
    return std::max(t1, start + d2);
}

// Piecewise-linear in t between measured points; the first point's value
// below it; the last segment's slope beyond the last point.
double g_predict_pts(const std::vector<std::pair<double, double>>& p, double t) {
    if (p.size() == 1) return p[0].second * t / p[0].first;
    if (t <= p[0].first) return p[0].second;
    for (size_t i = 1; i < p.size(); ++i) {
        if (t <= p[i].first) {
            const double t0 = p[i - 1].first, v0 = p[i - 1].second;
            const double t1 = p[i].first, v1 = p[i].second;
            return v0 + (v1 - v0) * (t - t0) / (t1 - t0);
        }
    }
    const double t0 = p[p.size() - 2].first, v0 = p[p.size() - 2].second;
    const double t1 = p.back().first, v1 = p.back().second;
    return v1 + (v1 - v0) * (t - t1) / (t1 - t0);
}

double g_predict(const TableKernel& k, double t) { return g_predict_pts(k.pts, t); }

int curve_set(const PerfTable& tab, const TableKernel& k, int64_t m) {
    const int classes = (int)tab.row_classes.size();
    const int64_t rows = ceil_div(m, k.uM);
    for (int i = 0; i < classes; ++i)
        if (rows <= tab.row_classes[i])
            return i < (int)k.by_rows.size() && !k.by_rows[i].pts.empty() ? i : classes;
    return classes;
}

const std::vector<std::pair<double, double>>& set_pts(const TableKernel& k, int set) {
    return set >= 0 && set < (int)k.by_rows.size() ? k.by_rows[set].pts : k.pts;
}

const std::vector<std::pair<double, double>>& set_tail(const TableKernel& k, int set, bool after_full) {
    if (set >= 0 && set < (int)k.by_rows.size()) return after_full ? k.by_rows[set].tailx : k.by_rows[set].tail;
    return after_full ? k.tailx : k.tail;
}

double tail_ratio(const std::vector<std::pair<double, double>>& p, double f) {
    if (p.empty() || f >= 1.0) return 1.0;
    if (f <= p[0].first) return p[0].second;
    for (size_t i = 1; i <= p.size(); ++i) {
        const double f1 = i < p.size() ? p[i].first : 1.0, r1 = i < p.size() ? p[i].second : 1.0;
        if (f <= f1) {
            const double f0 = p[i - 1].first, r0 = p[i - 1].second;
            return r0 + (r1 - r0) * (f - f0) / (f1 - f0);
        }
    }
    return 1.0;
}

double wave_fill(int64_t r, int64_t slots, int64_t cus) {
    if (r <= cus) return (double)r / (double)slots;
    return std::min(1.0, (double)(ceil_div(r, cus) * cus) / (double)slots);
}

double tail_ratio_tasks(const std::vector<std::pair<double, double>>& p, int64_t r, int64_t slots, int64_t cus) {
    const double f = wave_fill(r, slots, cus);
    if (f >= 1.0) return 1.0;
    double x0 = 0.0, y0 = 0.0;
    bool any = false;
    for (auto& q : p) {
        const double x = wave_fill(std::llround(q.first * (double)slots), slots, cus);
        if (x >= 1.0) break;   // this point and the later ones lie at a whole wave
        if (f <= x) return any ? y0 + (q.second - y0) * (f - x0) / (x - x0) : q.second;
        x0 = x;
        y0 = q.second;
        any = true;
    }
    return any ? y0 + (1.0 - y0) * (f - x0) / (1.0 - x0) : 1.0;
}

double wave_factor(const PerfTable& tab, const TableKernel& k, int64_t tasks, int set) {
    const int64_t slots = (int64_t)tab.cus * k.wg_per_cu;
    const int64_t full = tasks / slots, rem = tasks % slots;
    if (!rem) return (double)full;
    return (double)full + tail_ratio_tasks(set_tail(k, set, full > 0), rem, slots, tab.cus);
}

// Cost of one region served by one kernel with a requested split factor:
//   launch + (full waves + partial last wave) * g(steps) [+ split-K reduction]
// (with a kernel that has no tail points the wave term is ceil(tasks/slots),
// the page's f_wave).  A region of few tile rows takes g and the tail ratios
// from the kernel's curves for that many rows (curve_set).
double region_cost(const PerfTable& tab, int kernel, int64_t m, int64_t n, int64_t K, int64_t batch,
                   int s_req, Region* out) {
    const TableKernel& k = tab.kernels[kernel];
    const int64_t t3 = ceil_div(K, k.uK);
    const int64_t per = ceil_div(t3, s_req);
    const int64_t s_eff = ceil_div(t3, per);
    const int64_t tasks = ceil_div(m, k.uM) * ceil_div(n, k.uN) * s_eff * batch;
    const int64_t slots = (int64_t)tab.cus * k.wg_per_cu;
    const int64_t waves = ceil_div(tasks, slots);
    const int set = curve_set(tab, k, m);
    const double wf = wave_factor(tab, k, tasks, set);
    double c = tab.launch_us + wf * g_predict_pts(set_pts(k, set), (double)per);
    if (s_eff > 1)
        c += tab.red_launch_us + (double)(2 * s_eff + 1) * 4.0 * (double)m * (double)n * (double)batch /
                                     (tab.red_gbps * 1e3);
    if (out) {
        out->kernel = kernel;
        out->lib = k.lib_index;
        out->m = m;
        out->n = n;
        out->s = (int)s_eff;
        out->steps = (int)per;
        out->tasks = tasks;
        out->waves = waves;
        out->wave_factor = wf;
        out->cost = c;
    }
    return c;
}

namespace {

// Candidate strategies (MikPoly page, section 3 polymerization patterns;
// GPU uses patterns I and II):
//   I    : one region, one kernel, the whole M x N.
//   II-M : rows [0, cut) on kernel a, rows [cut, M) on kernel b != a, where
//          the cut is any multiple of uM(a) strictly inside M (region 1 is
//          tile-aligned; region 2 carries the ragged edge).  In the case
//          study region 1 is 3072 rows of kernel A: 96 of A's 108 slots.
//   II-N : the same along N.
// Every region takes its own split factor.  The search visits Pattern I
// first (a tight bound), then the II cuts in increasing order, skipping a
// cut whose region-1 cost plus a lower bound for region 2 reaches the best
// found, and stopping once no larger cut can win.  The best region 2 for a
// remaining extent e depends on e only (and on which kernel region 1 uses),
// so it is computed once per e and kept.
struct Searcher {
    const PerfTable& tab;
    const SearchOptions& opt;
    int64_t batch, M, N, K;
    int64_t evaluated = 0;

    // Curve sets: one per tile-row class of the table, then the square one.
    // Per kernel, a class whose curves it lacks maps to the square set.
    static constexpr int kSets = 8;
    int nclass = 0;   // row classes; set index nclass = square
    // g per row class (the square g for a class the kernel lacks, and at
    // index nclass), and the smallest g of the sets a region of that class
    // or more rows can take
    struct SplitChoice {
        int s_eff;
        int per;
        std::array<double, kSets> g, glb;
    };
    struct Floors {
        double tmin_alone = 1.0, tmin_after = 1.0;   // smallest partial-wave ratio (tail, tailx)
        double rho = 1.0;                            // smallest partial-wave ratio per filled slot
        double gmin = std::numeric_limits<double>::infinity();    // smallest g over the splits
        double sgmin = std::numeric_limits<double>::infinity();   // smallest s * g over the splits
        void merge(const Floors& o) {
            tmin_alone = std::min(tmin_alone, o.tmin_alone);
            tmin_after = std::min(tmin_after, o.tmin_after);
            rho = std::min(rho, o.rho);
            gmin = std::min(gmin, o.gmin);
            sgmin = std::min(sgmin, o.sgmin);
        }
    };
    std::vector<std::vector<SplitChoice>> sc;   // per kernel: distinct usable splits
    std::vector<double> min_g;                   // per kernel: cheapest single (possibly partial) wave
    std::vector<double> rate;                    // per kernel: lowest cost per output element
    // per kernel and row class: bounds of that class's curves (fl), and of
    // every set a region of that class or more rows may take (fls)
    std::vector<std::array<Floors, kSets>> fl, fls;
    std::vector<std::array<int8_t, kSets>> set_map;   // per kernel: row class -> curve set
    // per kernel and row class: the tail and tailx points with their fills
    // taken through wave_fill (points at a whole wave dropped)
    std::vector<std::array<std::array<std::vector<std::pair<double, double>>, 2>, kSets>> tails;
    std::vector<int8_t> class_by_rows;                // tile rows (up to the largest class) -> row class
    std::vector<FastDiv> dm, dn, dslots;         // per kernel: uM, uN and its slots as dividers
    double lb_region = 0.0;                      // lower bound of any region's cost
    double min_rate = 0.0;                       // lowest rate over allowed kernels

    Searcher(const PerfTable& t, const SearchOptions& o, int64_t b, int64_t m, int64_t n, int64_t k)
        : tab(t), opt(o), batch(b), M(m), N(n), K(k) {
        std::vector<int> req;
        if (opt.force_splitk > 0) {
            req.push_back(opt.force_splitk);
        } else {
            for (int s : tab.splits)
                if (s <= opt.splitk_max) req.push_back(s);
            if (req.empty()) req.push_back(1);
        }
        const size_t nk = tab.kernels.size();
        sc.resize(nk);
        min_g.assign(nk, std::numeric_limits<double>::infinity());
        rate.assign(nk, std::numeric_limits<double>::infinity());
        nclass = std::min<int>((int)tab.row_classes.size(), kSets - 1);
        if (nclass > 0) {
            class_by_rows.assign((size_t)tab.row_classes[nclass - 1] + 1, 0);
            for (int r = 0, c = 0; r <= tab.row_classes[nclass - 1]; ++r) {
                while (r > tab.row_classes[c]) ++c;
                class_by_rows[(size_t)r] = (int8_t)c;
            }
        }
        fl.assign(nk, {});
        fls.assign(nk, {});
        set_map.assign(nk, {});
        tails.assign(nk, {});
        dm.resize(nk);
        dn.resize(nk);
        dslots.resize(nk);
        lb_region = std::numeric_limits<double>::infinity();
        min_rate = std::numeric_limits<double>::infinity();
        for (size_t ki = 0; ki < nk; ++ki) {
            if (!kernel_allowed((int)ki)) continue;   // never scored
            const TableKernel& kk = tab.kernels[ki];
            const int64_t t3 = ceil_div(K, kk.uK);
            sc[ki].reserve(req.size());
            dm[ki].set(kk.uM);
            dn[ki].set(kk.uN);
            dslots[ki].set((int64_t)tab.cus * kk.wg_per_cu);
            for (int c = 0; c <= nclass; ++c)
                set_map[ki][c] = (int8_t)(c < nclass && c < (int)kk.by_rows.size() && !kk.by_rows[c].pts.empty()
                                              ? c : nclass);
            // a region's wave factor is at least tmin (one possibly partial
            // wave) and at least rho * tasks/slots (piecewise-linear ratios:
            // r(f)/f is smallest at a point or at f = 1; the wave's fill
            // through wave_fill is never below tasks/slots)
            const int64_t kslots = (int64_t)tab.cus * kk.wg_per_cu;
            for (int c = 0; c <= nclass; ++c) {
                Floors& f = fl[ki][c];
                for (int after = 0; after < 2; ++after) {
                    auto& dst = tails[ki][c][after];
                    for (auto& p : set_tail(kk, set_map[ki][c] < nclass ? set_map[ki][c] : -1, after)) {
                        const double x = wave_fill(std::llround(p.first * (double)kslots), kslots, tab.cus);
                        if (x >= 1.0) break;
                        dst.emplace_back(x, p.second);
                        (after ? f.tmin_after : f.tmin_alone) = std::min(after ? f.tmin_after : f.tmin_alone, p.second);
                        f.rho = std::min(f.rho, p.second / x);
                    }
                }
            }
            for (int s_req : req) {
                // a factor above the K-step count is only kept when forced
                if (s_req > 1 && s_req > t3 && opt.force_splitk <= 0) continue;
                const int64_t sr = std::min<int64_t>(s_req, std::max<int64_t>(t3, 1));
                const int64_t per = ceil_div(t3, sr);
                const int s_eff = (int)ceil_div(t3, per);
                bool dup = false;
                for (auto& c : sc[ki]) dup |= c.s_eff == s_eff;
                if (dup) continue;
                SplitChoice ch{s_eff, (int)per, {}, {}};
                ch.g[nclass] = g_predict(kk, (double)per);
                for (int c = 0; c < nclass; ++c)
                    ch.g[c] = set_map[ki][c] < nclass ? g_predict_pts(kk.by_rows[c].pts, (double)per) : ch.g[nclass];
                ch.glb[nclass] = ch.g[nclass];
                for (int c = nclass - 1; c >= 0; --c) ch.glb[c] = std::min(ch.g[c], ch.glb[c + 1]);
                sc[ki].push_back(ch);
                for (int c = 0; c <= nclass; ++c) {
                    Floors& f = fl[ki][c];
                    f.gmin = std::min(f.gmin, ch.g[c]);
                    f.sgmin = std::min(f.sgmin, (double)s_eff * ch.g[c]);
                }
            }
            // a region of class c or more rows takes one of the sets of
            // classes c, c+1, ... or the square one
            fls[ki][nclass] = fl[ki][nclass];
            for (int c = nclass - 1; c >= 0; --c) {
                fls[ki][c] = fl[ki][c];
                fls[ki][c].merge(fls[ki][c + 1]);
            }
            const Floors& f = fls[ki][0];   // every set
            const double slots = (double)tab.cus * kk.wg_per_cu;
            for (const SplitChoice& ch : sc[ki]) {
                min_g[ki] = std::min(min_g[ki], f.tmin_alone * ch.glb[0]);
                rate[ki] = std::min(rate[ki], f.rho * (double)ch.s_eff * ch.glb[0] / (slots * kk.uM * kk.uN));
            }
            lb_region = std::min(lb_region, tab.launch_us + min_g[ki]);
            min_rate = std::min(min_rate, rate[ki]);
        }
    }

    bool kernel_allowed(int k) const {
        return tab.kernels[k].bt == opt.bt && (!opt.conv || tab.kernels[k].conv_ok) &&
               (opt.force_kernel < 0 || opt.force_kernel == k);
    }

    double red_cost(int s_eff, int64_t m, int64_t n) const {
        return s_eff > 1 ? tab.red_launch_us +
                               (double)(2 * s_eff + 1) * 4.0 * (double)m * (double)n * (double)batch / (tab.red_gbps * 1e3)
                         : 0.0;
    }

    int64_t tiles_of(int k, int64_t m, int64_t n) const { return dm[k].ceil(m) * dn[k].ceil(n); }

    // tail_ratio_tasks over points already taken through wave_fill
    static double prepared_ratio(const std::vector<std::pair<double, double>>& p, double f) {
        if (f >= 1.0) return 1.0;
        if (p.empty()) return 1.0;
        if (f <= p[0].first) return p[0].second;
        for (size_t i = 1; i < p.size(); ++i)
            if (f <= p[i].first)
                return p[i - 1].second + (p[i].second - p[i - 1].second) * (f - p[i - 1].first) / (p[i].first - p[i - 1].first);
        return p.back().second + (1.0 - p.back().second) * (f - p.back().first) / (1.0 - p.back().first);
    }

    // Row class of an m-row region on kernel k (nclass: above every class);
    // it never falls as the region grows.
    int class_of(int k, int64_t m) const {
        if (nclass == 0) return 0;
        const int64_t rows = dm[k].ceil(m);
        return rows < (int64_t)class_by_rows.size() ? class_by_rows[(size_t)rows] : nclass;
    }
    // The curve set that prices it (as curve_set).
    int set_of(int k, int64_t m) const { return set_map[k][class_of(k, m)]; }
    double g_of(int k, const SplitChoice& c, int64_t m) const { return c.g[class_of(k, m)]; }

    double cost(int ki, const SplitChoice& c, int64_t m, int64_t n, Region* r) {
        ++evaluated;
        const TableKernel& k = tab.kernels[ki];
        const int64_t tasks = tiles_of(ki, m, n) * c.s_eff * batch;
        const int64_t slots = dslots[ki].d;
        int64_t rem;
        const int64_t full = dslots[ki].quot(tasks, rem);
        const int64_t waves = full + (rem != 0);
        const int cls = class_of(ki, m);
        const double g = c.g[cls];
        // full waves plus the partial last one (as wave_factor)
        const double wf = rem ? (double)full + prepared_ratio(tails[ki][cls][full > 0], wave_fill(rem, slots, tab.cus))
                              : (double)full;
        double v = tab.launch_us;
        if (opt.cost_mode == COST_WAVE) v += (double)waves;   // the page's f_wave alone
        else if (opt.cost_mode == COST_PIPE) v += g;
        else v += wf * g;
        v += red_cost(c.s_eff, m, n);
        if (r) {
            r->kernel = ki;
            r->lib = k.lib_index;
            r->m = m;
            r->n = n;
            r->s = c.s_eff;
            r->steps = c.per;
            r->tasks = tasks;
            r->waves = waves;
            r->wave_factor = wf;
            r->cost = v;
        }
        return v;
    }

    // Lower bound of the cost of region 1 on kernel a with split c for every
    // cut of at least m x n (a larger cut has at least as many full waves,
    // a partial wave costs at least the kernel's smallest tail ratio, and
    // the reduction grows with the area).
    // With lin, also the bound from the wave factor's linear floor, rho *
    // tasks/slots, which grows with the cut at least at the kernel's
    // lowest cost per output element.  A larger region may be of a higher
    // row class, so every set from this class on is bounded together.
    double lb_from(int a, const SplitChoice& c, int64_t m, int64_t n, double* lin = nullptr) const {
        const int64_t tasks = tiles_of(a, m, n) * c.s_eff * batch;
        int64_t rem;
        const int64_t full = dslots[a].quot(tasks, rem);
        const int cls = class_of(a, m);
        const Floors& f = fls[a][cls];
        const double g = c.glb[cls];
        const double part = rem ? (full ? f.tmin_after : f.tmin_alone) : 0.0;
        const double red = red_cost(c.s_eff, m, n);
        if (lin) *lin = tab.launch_us + f.rho * (double)tasks * dslots[a].inv * g + red;
        return tab.launch_us + ((double)full + part) * g + red;
    }

    // Lower bound of any region 2 of m x n.
    double lb2(int64_t m, int64_t n) const {
        return tab.launch_us + std::max((double)m * (double)n * (double)batch * min_rate, lb_region - tab.launch_us);
    }

    // Lower bound of an m x n region on kernel k with split c: its wave
    // factor is at least the smallest partial-wave ratio and at least rho
    // times tasks/slots.
    double lb_split(int k, const SplitChoice& c, int64_t tiles, int64_t m, int64_t n) const {
        const int cls = class_of(k, m);
        const Floors& f = fl[k][cls];
        const double w = std::max(f.tmin_alone, f.rho * (double)(tiles * c.s_eff * batch) * dslots[k].inv);
        return tab.launch_us + w * c.g[cls] + red_cost(c.s_eff, m, n);
    }
    // ... and over all of k's splits (s >= 1, no reduction term).
    double lb_kernel(int k, int64_t m, int64_t n) const {
        const double tiles = (double)(tiles_of(k, m, n) * batch);
        const Floors& f = fl[k][class_of(k, m)];
        return tab.launch_us + std::max(f.tmin_alone * f.gmin, f.rho * tiles * f.sgmin * dslots[k].inv);
    }

    // Both regions of a Pattern II cut in one launch over a kernel pair:
    // launch + the merged-wave makespan of the two task lists (each task as
    // long as its kernel's full-wave time g) + each region's split-K
    // reduction.  Not additive over the regions.
    double fused_cost(int a, const SplitChoice& c1, int64_t m1, int64_t n1, int b, const SplitChoice& c2,
                      int64_t m2, int64_t n2, Region* r1, Region* r2) {
        (void)cost(a, c1, m1, n1, r1);
        (void)cost(b, c2, m2, n2, r2);
        const TableKernel& ka = tab.kernels[a];
        const int64_t S = (int64_t)tab.cus * ka.wg_per_cu;
        return tab.launch_us + merged_makespan(S, r1->tasks, g_of(a, c1, m1), r2->tasks, g_of(b, c2, m2)) +
               red_cost(r1->s, r1->m, r1->n) +
               red_cost(r2->s, r2->m, r2->n);
    }

    bool fuse_allowed() const {
        return opt.fuse && opt.cost_mode == COST_FULL && opt.force_kernel < 0 && opt.allow_II && !tab.pairs.empty();
    }

    // Visit every one-launch Pattern II candidate: for each kernel pair
    // (a, b), direction, split of a, tile-aligned cut (as for Pattern II)
    // and split of b.  fn(cost, r1, r2, dir) sees each; it returns true when
    // the candidate became the best so far.  With use_bound, candidates
    // whose lower bound reaches `bound` are skipped: the makespan is at
    // least the first region's own waves, ceil(n1/S) d1 (which only grows
    // with the cut, as does its reduction), and at least the total work over
    // the slots.
    template <class F>
    void fused_candidates(double bound, bool use_bound, F&& fn) {
        for (auto& pr : tab.pairs) {
            const int a = pr.first, b = pr.second;
            if (!kernel_allowed(a) || !kernel_allowed(b)) continue;
            const TableKernel& ka = tab.kernels[a];
            const TableKernel& kb = tab.kernels[b];
            const int64_t S = (int64_t)tab.cus * ka.wg_per_cu;
            for (int dir = 0; dir < 2; ++dir) {
                if (dir == 0 && !tab.pat_IIM) continue;
                if (dir == 1 && !tab.pat_IIN) continue;
                const int64_t ext = dir == 0 ? M : N;
                const int64_t step = dir == 0 ? ka.uM : ka.uN;
                for (auto& c1s : sc[a]) {
                    for (int64_t cut = step; cut < ext; cut += step) {
                        const int64_t m1 = dir == 0 ? cut : M, n1 = dir == 0 ? N : cut;
                        const int64_t m2 = dir == 0 ? M - cut : M, n2 = dir == 0 ? N : N - cut;
                        const int64_t t1 = ceil_div(m1, ka.uM) * ceil_div(n1, ka.uN) * c1s.s_eff * batch;
                        const double g1 = g_of(a, c1s, m1);
                        const double own1 = (double)ceil_div(t1, S) * g1;
                        const double red1 = red_cost(c1s.s_eff, m1, n1);
                        // every larger cut: the smallest g of the sets it may take
                        const double own1_lb = (double)ceil_div(t1, S) * c1s.glb[class_of(a, m1)];
                        if (use_bound && tab.launch_us + own1_lb + red1 >= bound) break;
                        for (auto& c2s : sc[b]) {
                            const int64_t t2 = ceil_div(m2, kb.uM) * ceil_div(n2, kb.uN) * c2s.s_eff * batch;
                            const double lbv = tab.launch_us + red1 + red_cost(c2s.s_eff, m2, n2) +
                                               std::max(own1, ((double)t1 * g1 + (double)t2 * g_of(b, c2s, m2)) / (double)S);
                            if (use_bound && lbv >= bound) continue;
                            Region r1, r2;
                            const double v = fused_cost(a, c1s, m1, n1, b, c2s, m2, n2, &r1, &r2);
                            r1.m0 = r1.n0 = 0;
                            r2.m0 = dir == 0 ? cut : 0;
                            r2.n0 = dir == 0 ? 0 : cut;
                            if (fn(v, r1, r2, dir)) bound = std::min(bound, v);
                        }
                    }
                }
            }
        }
    }

    double best_region(int ki, int64_t m, int64_t n, Region* r) {
        double best = std::numeric_limits<double>::infinity();
        for (auto& c : sc[ki]) {
            Region tmp;
            const double v = cost(ki, c, m, n, &tmp);
            if (v < best) {
                best = v;
                *r = tmp;
            }
        }
        return best;
    }

    // The cheapest split of kernel k for an m x n region among those whose
    // cost is below thr (infinity and r untouched when none is).
    double best_region_below(int k, int64_t m, int64_t n, double thr, Region* r) {
        const int64_t tiles = tiles_of(k, m, n);
        double best = std::numeric_limits<double>::infinity();
        for (auto& c : sc[k]) {
            if (lb_split(k, c, tiles, m, n) >= std::min(thr, best)) continue;
            Region tmp;
            const double v = cost(k, c, m, n, &tmp);
            if (v < best && v < thr) {
                best = v;
                *r = tmp;
            }
        }
        return best;
    }

    // Best region 2 for one remaining extent: the cheapest kernel and split,
    // and the cheapest on a different kernel (region 2 may not reuse region
    // 1's kernel), both only among regions cheaper than thr -- a kernel or
    // split whose lower bound reaches thr is not scored.  Kernels are
    // visited in table order, so ties keep the earliest, as in a plain scan.
    struct Second {
        double c1 = std::numeric_limits<double>::infinity(), c2 = std::numeric_limits<double>::infinity();
        Region r1, r2;
        double thr = -1.0;   // exact for every cost below thr
    };
    Second second_for(int64_t m, int64_t n, double thr = std::numeric_limits<double>::infinity()) {
        Second out;
        out.thr = thr;
        const int nk = (int)tab.kernels.size();
        for (int b = 0; b < nk; ++b) {
            if (!kernel_allowed(b)) continue;
            if (lb_kernel(b, m, n) >= thr) continue;
            Region r;
            const double v = best_region_below(b, m, n, thr, &r);
            if (!(v < thr)) continue;
            if (v < out.c1) {
                if (out.r1.kernel >= 0 && out.r1.kernel != b) {
                    out.c2 = out.c1;
                    out.r2 = out.r1;
                }
                out.c1 = v;
                out.r1 = r;
            } else if (v < out.c2 && b != out.r1.kernel) {
                out.c2 = v;
                out.r2 = r;
            }
        }
        return out;
    }

    // The bounds below hold for the full model only; the ablations and the
    // ranked list score every candidate.
    bool prune() const { return !opt.exhaustive && opt.cost_mode == COST_FULL; }

    // Every candidate of the space (each region with each of its splits),
    // ordered by modelled cost (ties keep enumeration order); returns the
    // rank-th (1-based) and the size of the space.  Only the `rank` cheapest
    // are kept while the space is walked.
    Plan ranked(int rank) {
        struct Cand {
            double cost;
            int64_t seq;
            int pattern;
            Region r1, r2;
            bool fused = false;
        };
        auto worse = [](const Cand& x, const Cand& y) { return x.cost < y.cost || (x.cost == y.cost && x.seq < y.seq); };
        std::vector<Cand> heap;   // max-heap under `worse`: the worst kept candidate on top
        int64_t seq = 0;
        auto offer = [&](Cand&& x) {
            x.seq = seq++;
            if ((int64_t)heap.size() < rank) {
                heap.push_back(std::move(x));
                std::push_heap(heap.begin(), heap.end(), worse);
            } else if (!heap.empty() && worse(x, heap.front())) {
                std::pop_heap(heap.begin(), heap.end(), worse);
                heap.back() = std::move(x);
                std::push_heap(heap.begin(), heap.end(), worse);
            }
        };
        const int nk = (int)tab.kernels.size();
        if (tab.pat_I)
            for (int a = 0; a < nk; ++a) {
                if (!kernel_allowed(a)) continue;
                for (auto& c : sc[a]) {
                    Cand x{0.0, 0, PAT_I, {}, {}};
                    x.cost = cost(a, c, M, N, &x.r1);
                    offer(std::move(x));
                }
            }
        if (opt.force_kernel < 0 && opt.allow_II)
            for (int dir = 0; dir < 2; ++dir) {
                if (dir == 0 && !tab.pat_IIM) continue;
                if (dir == 1 && !tab.pat_IIN) continue;
                const int64_t ext = dir == 0 ? M : N;
                for (int a = 0; a < nk; ++a) {
                    if (!kernel_allowed(a)) continue;
                    const TableKernel& ka = tab.kernels[a];
                    const int64_t step = dir == 0 ? ka.uM : ka.uN;
                    for (auto& c1s : sc[a]) {
                        for (int64_t cut = step; cut < ext; cut += step) {
                            const int64_t m1 = dir == 0 ? cut : M, n1 = dir == 0 ? N : cut;
                            const int64_t m2 = dir == 0 ? M - cut : M, n2 = dir == 0 ? N : N - cut;
                            Region r1;
                            const double c1 = cost(a, c1s, m1, n1, &r1);
                            for (int b = 0; b < nk; ++b) {
                                if (b == a || !kernel_allowed(b)) continue;
                                for (auto& c2s : sc[b]) {
                                    Cand x{0.0, 0, dir == 0 ? PAT_IIM : PAT_IIN, r1, {}};
                                    x.cost = c1 + cost(b, c2s, m2, n2, &x.r2);
                                    x.r2.m0 = dir == 0 ? cut : 0;
                                    x.r2.n0 = dir == 0 ? 0 : cut;
                                    offer(std::move(x));
                                }
                            }
                        }
                    }
                }
            }
        if (fuse_allowed())
            fused_candidates(0.0, false, [&](double v, const Region& r1, const Region& r2, int dir) {
                offer(Cand{v, 0, dir == 0 ? PAT_IIM : PAT_IIN, r1, r2, true});
                return false;
            });
        Plan p;
        p.rank = rank;
        p.candidates = seq;
        if (rank < 1 || rank > (int64_t)heap.size()) {
            p.pattern = PAT_I;
            p.cost_us = std::numeric_limits<double>::infinity();
            return p;   // no regions: the caller reports "no plan"
        }
        std::sort_heap(heap.begin(), heap.end(), worse);
        const Cand& c = heap[rank - 1];
        p.pattern = c.pattern;
        p.cost_us = c.cost;
        p.fused = c.fused;
        p.regions.push_back(c.r1);
        if (c.pattern != PAT_I) p.regions.push_back(c.r2);
        p.regions[0].m0 = p.regions[0].n0 = 0;
        return p;
    }

    Plan run() {
        if (opt.plan_rank > 0) return ranked(opt.plan_rank);
        Plan best;
        best.cost_us = prune() && opt.bound < 1e300 ? opt.bound : std::numeric_limits<double>::infinity();
        const int nk = (int)tab.kernels.size();
        if (tab.pat_I) {
            for (int a = 0; a < nk; ++a) {
                if (!kernel_allowed(a)) continue;
                Region r;
                const double c = best_region(a, M, N, &r);
                if (c < best.cost_us) {
                    best.pattern = PAT_I;
                    best.cost_us = c;
                    r.m0 = r.n0 = 0;
                    best.regions.assign(1, r);
                }
            }
        }
        if (opt.force_kernel >= 0 || !opt.allow_II) {
            if (best.regions.empty()) best.cost_us = std::numeric_limits<double>::infinity();
            return best;
        }
        // any Pattern II plan costs at least two launches plus the whole
        // output at the cheapest rate per element of any kernel
        const bool II_hopeless =
            prune() && 2.0 * tab.launch_us + (double)M * (double)N * (double)batch * min_rate >= best.cost_us;
        for (int dir = 0; dir < 2 && !II_hopeless; ++dir) {
            if (dir == 0 && !tab.pat_IIM) continue;
            if (dir == 1 && !tab.pat_IIN) continue;
            const int64_t ext = dir == 0 ? M : N;
            // remaining extent -> best region 2; every cut is a multiple of
            // the gcd of the allowed kernels' steps, so cut / gcd indexes it
            int64_t gstep = 0;
            for (int a = 0; a < nk; ++a)
                if (kernel_allowed(a)) gstep = std::gcd(gstep, (int64_t)(dir == 0 ? tab.kernels[a].uM : tab.kernels[a].uN));
            if (gstep <= 0 || gstep >= ext) continue;
            std::vector<int32_t> slot((size_t)(ext / gstep) + 1, -1);
            std::vector<Second> seconds;
            std::vector<char> dead;
            for (int a = 0; a < nk; ++a) {
                if (!kernel_allowed(a)) continue;
                const TableKernel& ka = tab.kernels[a];
                const int64_t step = dir == 0 ? ka.uM : ka.uN;
                const std::vector<SplitChoice>& splits = sc[a];
                dead.assign(splits.size(), 0);
                size_t live = splits.size();
                for (int64_t cut = step; cut < ext && live > 0; cut += step) {
                    const int64_t e = ext - cut;
                    const int64_t m1 = dir == 0 ? cut : M, n1 = dir == 0 ? N : cut;
                    const int64_t m2 = dir == 0 ? e : M, n2 = dir == 0 ? N : e;
                    // region 1: the cheapest split at this cut; a split whose
                    // bound for this and every larger cut reaches the best
                    // plan is dropped for good
                    double c1 = std::numeric_limits<double>::infinity();
                    Region r1;
                    const double l2 = prune() ? lb2(m2, n2) : 0.0;
                    for (size_t i = 0; i < splits.size(); ++i) {
                        if (dead[i]) continue;
                        if (prune()) {
                            double lin;
                            const double lb = lb_from(a, splits[i], m1, n1, &lin);
                            // lin + lb2 never falls as the cut grows: region
                            // 1 gains at least min_rate per element it takes
                            // from region 2
                            if (lb + lb_region >= best.cost_us || lin + l2 >= best.cost_us) {
                                dead[i] = 1;
                                --live;
                                continue;
                            }
                            if (lb + l2 >= best.cost_us) continue;
                        }
                        Region r;
                        const double v = cost(a, splits[i], m1, n1, &r);
                        if (v < c1) {
                            c1 = v;
                            r1 = r;
                        }
                    }
                    if (!(c1 < best.cost_us)) continue;
                    if (prune() && c1 + lb2(m2, n2) >= best.cost_us) continue;
                    // region 2 only matters below best - c1: score it to that
                    // bound, once per extent (again if a later cut asks for a
                    // higher bound)
                    const double thr = prune() ? best.cost_us - c1 : std::numeric_limits<double>::infinity();
                    int32_t& si = slot[(size_t)(cut / gstep)];
                    if (si < 0) {
                        si = (int32_t)seconds.size();
                        seconds.push_back(second_for(m2, n2, thr));
                    } else if (seconds[si].thr < thr) {
                        seconds[si] = second_for(m2, n2, thr);
                    }
                    const Second& sd = seconds[si];
                    const bool own = sd.r1.kernel == a;
                    const double c2 = own ? sd.c2 : sd.c1;
                    if (!(c1 + c2 < best.cost_us)) continue;
                    Region r2 = own ? sd.r2 : sd.r1;
                    best.pattern = dir == 0 ? PAT_IIM : PAT_IIN;
                    best.cost_us = c1 + c2;
                    r1.m0 = r1.n0 = 0;
                    r2.m0 = dir == 0 ? cut : 0;
                    r2.n0 = dir == 0 ? 0 : cut;
                    best.regions.assign({r1, r2});
                }
            }
        }
        // one-launch Pattern II over kernel pairs (not additive: scored
        // whole, bounded by the first region's full waves)
        if (fuse_allowed())
            fused_candidates(best.cost_us, prune(), [&](double v, const Region& r1, const Region& r2, int dir) {
                if (!(v < best.cost_us)) return false;
                best.pattern = dir == 0 ? PAT_IIM : PAT_IIN;
                best.cost_us = v;
                best.fused = true;
                best.regions.assign({r1, r2});
                return true;
            });
        if (best.regions.empty()) best.cost_us = std::numeric_limits<double>::infinity();
        return best;
    }
};

}  // namespace

Plan polymerize(const PerfTable& tab, int64_t batch, int64_t M, int64_t N, int64_t K,
                const SearchOptions& opt) {
    auto t0 = std::chrono::steady_clock::now();
    Plan p;
    if (batch == 0 || M == 0 || N == 0) {
        p.pattern = PAT_EMPTY;
    } else if (K == 0) {
        p.pattern = PAT_ZERO;
    } else {
        Searcher s(tab, opt, batch, M, N, K);
        p = s.run();
        p.evaluated = s.evaluated;
    }
    auto t1 = std::chrono::steady_clock::now();
    p.plan_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
    return p;
}

Plan polymerize_grouped(const PerfTable& tab, int64_t M, int64_t K, const std::vector<int64_t>& Ns,
                        const SearchOptions& opt) {
    auto t0 = std::chrono::steady_clock::now();
    Plan best;
    best.pattern = PAT_I;
    best.cost_us = std::numeric_limits<double>::infinity();
    int64_t Nsum = 0;
    for (int64_t n : Ns) Nsum += n;
    std::vector<int> req;
    if (opt.force_splitk > 0) {
        req.push_back(opt.force_splitk);
    } else {
        for (int s : tab.splits)
            if (s <= opt.splitk_max) req.push_back(s);
        if (req.empty()) req.push_back(1);
    }
    for (size_t ki = 0; ki < tab.kernels.size(); ++ki) {
        const TableKernel& k = tab.kernels[ki];
        if (k.bt != opt.bt || (opt.force_kernel >= 0 && opt.force_kernel != (int)ki)) continue;
        const int64_t t3 = ceil_div(K, k.uK);
        int64_t cols = 0;
        for (int64_t n : Ns) cols += ceil_div(n, k.uN);
        const int64_t slots = (int64_t)tab.cus * k.wg_per_cu;
        for (int s_req : req) {
            if (s_req > 1 && s_req > t3 && opt.force_splitk <= 0) continue;
            const int64_t sr = std::min<int64_t>(s_req, std::max<int64_t>(t3, 1));
            const int64_t per = ceil_div(t3, sr);
            const int64_t s_eff = ceil_div(t3, per);
            const int64_t tasks = ceil_div(M, k.uM) * cols * s_eff;
            const int set = curve_set(tab, k, M);
            const double wf = wave_factor(tab, k, tasks, set);
            double c = tab.launch_us + wf * g_predict_pts(set_pts(k, set), (double)per);
            if (s_eff > 1)
                for (int64_t n : Ns)
                    c += tab.red_launch_us + (double)(2 * s_eff + 1) * 4.0 * (double)M * (double)n / (tab.red_gbps * 1e3);
            ++best.evaluated;
            if (c < best.cost_us) {
                Region r;
                r.m = M;
                r.n = Nsum;
                r.kernel = (int)ki;
                r.lib = k.lib_index;
                r.s = (int)s_eff;
                r.steps = (int)per;
                r.tasks = tasks;
                r.waves = ceil_div(tasks, slots);
                r.wave_factor = wf;
                r.cost = c;
                best.cost_us = c;
                best.regions.assign(1, r);
            }
        }
    }
    auto t1 = std::chrono::steady_clock::now();
    best.plan_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
    return best;
}

double transpose_cost(const PerfTable& tab, int64_t batch, int64_t N, int64_t K) {
    if (!(tab.tr_gbps > 0)) return std::numeric_limits<double>::infinity();
    return tab.tr_launch_us + 4.0 * (double)K * (double)N * (double)batch / (tab.tr_gbps * 1e3);
}

Plan plan_call(const PerfTable& tab, int64_t batch, int64_t M, int64_t N, int64_t K, const SearchOptions& opt,
               int transpose_mode) {
    Plan p = polymerize(tab, batch, M, N, K, opt);
    if (opt.bt || transpose_mode == 0 || p.pattern == PAT_EMPTY || p.pattern == PAT_ZERO || opt.plan_rank > 0 ||
        opt.force_kernel >= 0 || opt.cost_mode != COST_FULL)
        return p;
    double tc = transpose_cost(tab, batch, N, K);
    if (!std::isfinite(tc)) {
        if (transpose_mode != 2) return p;
        tc = 0.0;   // forced without figures: the copy goes unpriced
    }
    SearchOptions o = opt;
    o.bt = true;
    // only an N x K plan cheaper than the K x N one after paying for the copy matters
    if (transpose_mode != 2 && !p.regions.empty()) o.bound = std::min(o.bound, p.cost_us - tc);
    Plan q = polymerize(tab, batch, M, N, K, o);
    if (q.regions.empty() || !(transpose_mode == 2 || q.cost_us + tc < p.cost_us || p.regions.empty())) {
        p.plan_us += q.plan_us;
        p.evaluated += q.evaluated;
        return p;
    }
    q.transpose_b = true;
    q.transpose_us = tc;
    q.cost_us += tc;
    q.plan_us += p.plan_us;
    q.evaluated += p.evaluated;
    return q;
}

std::string plan_to_json(const Plan& p, const PerfTable& tab) {
    static const char* names[] = {"empty", "zero", "I", "II-M", "II-N"};
    std::ostringstream o;
    o.precision(17);
    o << "{\"pattern\":\"" << names[p.pattern] << "\",\"cost_us\":" << (p.regions.empty() ? 0.0 : p.cost_us)
      << ",\"plan_us\":" << p.plan_us << ",\"evaluated\":" << p.evaluated;
    if (p.rank > 0) o << ",\"rank\":" << p.rank << ",\"candidates\":" << p.candidates;
    o << ",\"transpose_b\":" << (p.transpose_b ? "true" : "false");
    o << ",\"fused\":" << (p.fused ? "true" : "false");
    if (p.transpose_b) o << ",\"transpose_us\":" << p.transpose_us;
    o << ",\"regions\":[";
    for (size_t i = 0; i < p.regions.size(); ++i) {
        const Region& r = p.regions[i];
        const TableKernel& k = tab.kernels[r.kernel];
        if (i) o << ",";
        o << "{\"m0\":" << r.m0 << ",\"n0\":" << r.n0 << ",\"m\":" << r.m << ",\"n\":" << r.n
          << ",\"kernel\":\"" << k.name << "\",\"uM\":" << k.uM << ",\"uN\":" << k.uN << ",\"uK\":" << k.uK
          << ",\"s\":" << r.s << ",\"steps\":" << r.steps << ",\"tasks\":" << r.tasks
          << ",\"waves\":" << r.waves << ",\"wave_factor\":" << r.wave_factor << ",\"cost_us\":" << r.cost << "}";
    }
    o << "]}";
    return o.str();
}

}  // namespace mkp
