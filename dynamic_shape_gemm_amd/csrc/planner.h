// Run-time polymerizer: performance table, cost model and strategy search.
//
// Pure host C++ (no HIP): it decides, for a GEMM shape known only at run
// time, how the output is cut into regions, which fixed-size micro-kernel
// serves each region and how many K splits each region uses.
//
// MikPoly page, section 3:
//  * "micro-kernel performance model": a task is one uM x uN output tile that
//    runs t = ceil(K/uK) micro-kernel instances back to back on one PE;
//    g_predict(t) is measured offline per micro-kernel.
//  * "polymerization cost model": Cost(S,H) = sum_i f_wave * f_pipe with
//    f_wave = ceil(f_parallel / |P_multi|), f_pipe = g_predict(f_num).
//  * "complete algorithm": candidate strategies whose partial cost already
//    reaches the best one found are skipped.
#pragma once

#include <cstdint>
#include <string>
#include <utility>
#include <vector>

namespace mkp {

// One kernel's curves measured on one wave layout.
struct Curves {
    std::vector<std::pair<double, double>> pts;           // (t, us), sorted by t; empty: not measured
    std::vector<std::pair<double, double>> tail, tailx;   // as TableKernel::tail, tailx
};

struct TableKernel {
    std::string name;
    int uM = 0, uN = 0, uK = 0;
    int wg_per_cu = 1;                               // resident workgroups per CU
    bool bt = false;                                 // serves B given as N x K
    std::vector<std::pair<double, double>> pts;      // (t, us), sorted by t
    // Partial last wave: (fraction f of the slots filled, time of that wave
    // relative to a full one), sorted by f; empty = every wave costs a full g.
    // `tail` holds a wave that runs alone (fewer tasks than slots); `tailx`
    // the extra time a partial wave adds after full waves, whose stragglers
    // it overlaps.
    std::vector<std::pair<double, double>> tail, tailx;
    // The same three curves measured on waves of few tile rows (the rest of
    // the slots filled by tile columns, at most 32, then by K splits):
    // by_rows[i] on a wave of PerfTable::row_classes[i] rows.  The curves
    // above are measured on a square wave.
    std::vector<Curves> by_rows;
    int lib_index = -1;                              // index in the kernel library, -1 if none
    bool conv_ok = false;                            // the library has a convolution form of it
};

struct PerfTable {
    int cus = 256;
    double launch_us = 0.0;       // per launch (per region)
    double red_launch_us = 0.0;   // split-K reduction: fixed part
    double red_gbps = 1000.0;     // split-K reduction: bandwidth
    // transposing a K x N B into an N x K copy (so that a K x N call can run
    // on the N x K kernels): fixed part and bandwidth; tr_gbps 0 = never
    double tr_launch_us = 0.0;
    double tr_gbps = 0.0;
    std::vector<int> splits{1};
    // Tile-row counts, ascending, with curves of their own: a region of r
    // tile rows takes the curves of the smallest class >= r when its kernel
    // has them, else the square ones.
    std::vector<int> row_classes;
    bool pat_I = true, pat_IIM = true, pat_IIN = true;
    double mfma_tflops = 0.0;     // measured sustained bf16 MFMA rate (0: unknown)
    double hbm_gbps = 0.0;        // measured streaming-copy bandwidth, read + write (0: unknown)
    double hbm_read_gbps = 0.0;   // measured read-only streaming bandwidth (0: unknown)
    std::vector<TableKernel> kernels;
    // Kernel pairs (indices into kernels) compiled into one launch: a Pattern
    // II plan over such a pair may run both regions in one launch.  Both
    // kernels of a pair share layout and resident workgroups per CU.
    std::vector<std::pair<int, int>> pairs;
};

enum PatternKind { PAT_EMPTY = 0, PAT_ZERO = 1, PAT_I = 2, PAT_IIM = 3, PAT_IIN = 4 };

struct Region {
    int64_t m0 = 0, n0 = 0, m = 0, n = 0;
    int kernel = -1;        // index into PerfTable::kernels
    int lib = -1;           // library kernel that serves it (-1: not launchable)
    int s = 1;              // K splits actually used
    int steps = 0;          // K steps (of uK) per split = f_num
    int64_t tasks = 0;      // f_parallel (includes splits and batch)
    int64_t waves = 0;      // f_wave = ceil(tasks / slots)
    double wave_factor = 0; // full waves + relative time of the partial last one
    double cost = 0.0;
};

struct Plan {
    int pattern = PAT_EMPTY;
    std::vector<Region> regions;
    double cost_us = 0.0;
    double plan_us = 0.0;
    int64_t evaluated = 0;   // candidate regions scored
    int rank = 0;            // >0: this is the rank-th cheapest candidate
    int64_t candidates = 0;  // size of the ranked candidate list (rank > 0 only)
    bool transpose_b = false;  // a K x N B is first copied to N x K; regions use N x K kernels
    double transpose_us = 0.0; // modelled time of that copy (included in cost_us)
    bool fused = false;        // the two regions run in one launch (a kernel pair)
};

// Which factors of the cost model the search scores (MikPoly page, section 5
// ablation): the full product f_wave * f_pipe, f_wave alone (f_pipe taken as
// 1 us), or f_pipe alone (f_wave taken as 1).  The launch and split-K
// reduction terms stay in all three.
enum CostMode { COST_FULL = 0, COST_WAVE = 1, COST_PIPE = 2 };

struct SearchOptions {
    bool exhaustive = false;
    int force_kernel = -1;   // table index; -1 = free choice
    int force_splitk = 0;    // 0 = free choice
    int splitk_max = 64;
    bool allow_II = true;
    int cost_mode = COST_FULL;
    int plan_rank = 0;       // >0: return the rank-th cheapest candidate of the whole space
    bool bt = false;         // B is N x K: only kernels of that layout take part
    bool fuse = false;       // consider one-launch Pattern II plans over kernel pairs
    bool conv = false;       // implicit-GEMM convolution: only kernels with a convolution form
    // only plans strictly cheaper than this are of interest (infinity: any);
    // when none is, the result has no regions
    double bound = 1e300;
};

// Parse the text form of a table.  Returns false and sets err on bad input.
bool parse_table(const std::string& text, PerfTable& out, std::string& err);
std::string table_to_text(const PerfTable& t);

double g_predict(const TableKernel& k, double t);
// g from an explicit list of (t, us) points (same interpolation).
double g_predict_pts(const std::vector<std::pair<double, double>>& pts, double t);
// Which curves price an m-row region on kernel k: an index into k.by_rows,
// or row_classes.size() for the square curves.
int curve_set(const PerfTable& tab, const TableKernel& k, int64_t m);
const std::vector<std::pair<double, double>>& set_pts(const TableKernel& k, int set);
const std::vector<std::pair<double, double>>& set_tail(const TableKernel& k, int set, bool after_full);
// Time of a wave whose tasks fill a fraction f (0 < f <= 1) of the slots,
// relative to a full wave: 1 without tail points; linear between points and
// up to (1, 1); the first point's value below it.
double tail_ratio(const std::vector<std::pair<double, double>>& pts, double f);
// The fill of a wave of r tasks on `slots` slots over `cus` CUs as its
// busiest CU sees it: workgroups are spread over the CUs before any CU takes
// a second, so up to one task per CU the fill is r/slots, and beyond it
// some CU holds ceil(r/cus) tasks, as in a wave of ceil(r/cus) * cus.
double wave_fill(int64_t r, int64_t slots, int64_t cus);
// tail_ratio of a wave of r tasks with the measured fills and r both taken
// through wave_fill (measured points at or past a whole wave drop out).
double tail_ratio_tasks(const std::vector<std::pair<double, double>>& pts, int64_t r, int64_t slots, int64_t cus);
// Waves a region of `tasks` tasks costs: full waves plus the partial last one.
double wave_factor(const PerfTable& tab, const TableKernel& k, int64_t tasks, int set = -1);
double region_cost(const PerfTable& tab, int kernel, int64_t m, int64_t n, int64_t K,
                   int64_t batch, int s_req, Region* out);

// Time to run n1 tasks of duration d1 and then n2 tasks of duration d2 on S
// slots, each task starting on the earliest free slot in that order (the
// merged-wave view of one launch holding two regions): the second region's
// tasks fill the slots the first region's last wave leaves free.  With
// d1 == d2 it is ceil((n1 + n2) / S) * d1.
double merged_makespan(int64_t S, int64_t n1, double d1, int64_t n2, double d2);

Plan polymerize(const PerfTable& tab, int64_t batch, int64_t M, int64_t N, int64_t K,
                const SearchOptions& opt);

// Grouped call C_g = A . B_g (g < G, shared A and K): Pattern I over the
// tile columns of all groups -- one kernel and one split factor, tasks =
// ceil(M/uM) * sum_g ceil(N_g/uN) * s, one launch, and with s > 1 one
// reduction per group.
Plan polymerize_grouped(const PerfTable& tab, int64_t M, int64_t K, const std::vector<int64_t>& Ns,
                        const SearchOptions& opt);

// Modelled time of transposing batch K x N bf16 matrices (reads and writes
// 2*K*N bytes each); infinite when the table has no transpose figures.
double transpose_cost(const PerfTable& tab, int64_t batch, int64_t N, int64_t K);

// The plan for a call: for B given as N x K the N x K search; for B given as
// K x N the cheaper of the K x N search and a transpose of B followed by the
// N x K search.  transpose_mode: 0 never transpose, 1 by modelled cost (when
// the table prices the copy), 2 always (when an N x K plan exists).
Plan plan_call(const PerfTable& tab, int64_t batch, int64_t M, int64_t N, int64_t K, const SearchOptions& opt,
               int transpose_mode);

std::string plan_to_json(const Plan& p, const PerfTable& tab);

}  // namespace mkp
