// Host-side view of the micro-kernel library: the argument block every
// micro-kernel takes and the registry of launchable instances.
//
// Each micro-kernel is a fixed uM x uN x uK tile (MikPoly page, section 3,
// "micro-kernel generation"); the region's start addresses, extents and K
// trip counts arrive as run-time scalars (section 4, GPU platform).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace mkp {

// flags bits
enum : int {
    KF_VEC_A = 1,   // A rows 16-byte aligned: 128-bit loads allowed
    KF_VEC_B = 2,   // B rows 16-byte aligned
    KF_VEC_C = 4,   // C rows 16-byte aligned: 128-bit stores allowed
    KF_VEC_COUT = 8,  // final C rows (fused split-K) 16-byte aligned
    KF_EPI = 16,      // apply the epilogue below to the final C values
    KF_CONV_DMA = 32, // convolution with C % uK == 0 (a K step stays in one filter tap) and every
                      // input offset, padding included, within 32 bits: direct loads
    KF_NT_C = 64,     // C (or the split-K partials) written with streaming (nontemporal) 16-byte stores
    KF_SC1_C = 128,   // ... written through to the level every XCD shares (sc1)
};

// Implicit-GEMM convolution (the MikPoly page runs convolutions as GEMMs):
// A is never stored.  Row m of A is output pixel (n, p, q) of an NHWC input
// and column k is filter tap (r, s) and input channel c, k = (r S + s) C + c;
// A(m, k) = x[n][p sh - ph + r dh][q sw - pw + s dw][c], zero outside the
// image.  B is the KRSC filter bank (an N x K matrix), C the NPQK output.
struct KConv {
    const uint16_t* zero;   // 16 zero bytes: where padded input is read from
    int m0;                 // first A row of the launch's region
    int H, W, C, S, P, Q;
    int sh, sw, ph, pw, dh, dw;
    int R;                  // filter height (bounds of the 32-bit direct-load offsets)
};

// Fused epilogue (Bolt page, epilogue fusion, and its persistent-kernel
// form D = alpha.A.W + beta.C): each final value becomes
//   act(alpha * acc + beta * C_old + bias[n]),
// C_old read from the output itself (only when beta != 0), bias indexed by
// the region's column.  Split-K partials never see it: the reduction does.
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2, ACT_GELU_TANH = 3, ACT_SILU = 4, ACT_COUNT = 5 };
struct KEpi {
    const float* bias;   // region column 0 of the bias vector, or null
    float alpha, beta;
    int act;
};

// One group of a grouped call: C_g = A . B_g over the tile columns
// [tile0, tile0 + ceil(N / uN)) of the launch (groups share A and K).
struct KGroup {
    const uint16_t* B;
    float* C;
    int64_t ldb, ldc;
    int N;
    int tile0;
    int flags;   // this group's KF_VEC_B / KF_VEC_C / KF_NT_C bits
};
enum : int { kMaxGroups = 4 };

struct KArgs {
    const uint16_t* A;    // region origin in A (row m0, column 0)
    const uint16_t* B;    // B (row 0, column 0 of a K x N matrix, or of an N x K one); the kernel adds n0
    float* C;             // region origin in C, or the split-K workspace
    int64_t lda, ldb, ldc;
    int64_t sA, sB, sC;   // batch strides (elements)
    int64_t sCsplit;      // elements between split partials (0 when s == 1)
    int M, N, K;          // region extents and full K
    int tiles_m, tiles_n;
    int steps_per_split;  // K steps of uK per split
    int splits;           // K splits (grid covers tiles x splits x batch)
    int batch;
    int flags;
    // Fused split-K reduction (splits > 1 and counters != nullptr): C above is
    // the partial workspace; the last split of a tile to finish sums the
    // partials in split order into Cout.  counters: one int per tile and batch
    // entry, zero before the launch and left zero after it.
    int* counters;
    float* Cout;
    int64_t ldcout, sCout;
    // Grouped call (ngroups > 0, batch 1, no fused reduction): tile columns
    // are dealt group after group; B, N and (with one split) C, ldc come from
    // the tile's group.  With several splits C above is the partial
    // workspace, whose columns follow the launch's tile columns.
    int ngroups;
    KGroup group[kMaxGroups];
    KEpi epi;             // used when flags has KF_EPI
    KConv conv;           // convolution kernels only: A is the NHWC input
};

struct KernelInfo {
    const char* name;
    int uM, uN, uK;
    int threads;
    int lds_bytes;
    bool fused_ok;        // compiled with the fused split-K reduction
    bool bt;              // B given as N x K (K-contiguous rows) instead of K x N
    const void* func;     // __global__ entry, for occupancy queries
    hipError_t (*launch)(const KArgs&, dim3 grid, hipStream_t);
};

// Launch timing: while a thread's slot holds two events, the next library
// launch on that thread records its kernel's own start and end in them
// (hipExtLaunchKernel: timestamps of the dispatch itself, not of the stream
// around it) and empties the slot.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

// The allocation-free entry point's device memory: kStaticScratchBytes at a
// 256-byte aligned address of device `dev` (which must be current), looked up
// on the first call for that device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(int dev, void** out);

int kernel_count();
const KernelInfo& kernel_info(int i);
int kernel_find(const char* name);

// A pair of micro-kernels compiled into one launch: the first `n1`
// workgroups run kernel `first` over one region, the others kernel `second`
// over another (grid = n1 + the second region's workgroups).
struct DualInfo {
    const char* first;
    const char* second;
    const void* func;
    hipError_t (*launch)(const KArgs& a1, const KArgs& a2, int n1, dim3 grid, hipStream_t);
};
int dual_count();
const DualInfo& dual_info(int i);

// The convolution form of an N x K micro-kernel (same tile; A gathered from
// an NHWC input through KArgs::conv).
struct ConvInfo {
    const char* twin;     // name of the N x K kernel with the same tile
    const void* func;
    hipError_t (*launch)(const KArgs&, dim3 grid, hipStream_t);
};
int conv_count();
const ConvInfo& conv_info(int i);

// Sum of `splits` partials W[z] (z ascending) into C; W is [splits][batch][M][ldw].
// With an epilogue (epi non-null) the sum goes through it; splits == 0 is an
// empty sum (W unused), which with the epilogue serves K == 0.  vec: bit 0,
// C rows 16-byte aligned (128-bit stores); bit 1, with bit 0, C written with
// streaming stores (as KF_NT_C).
hipError_t launch_splitk_reduce(const float* W, int splits, int64_t sWsplit, int64_t sWbatch, int64_t ldw,
                                float* C, int64_t ldc, int64_t sC, int M, int N, int batch, int vec,
                                hipStream_t st, const KEpi* epi = nullptr);
// C := 0 for batch matrices of M x N (K == 0: empty sum).
hipError_t launch_zero_fill(float* C, int64_t ldc, int64_t sC, int M, int N, int batch, hipStream_t st);

// Copy batch x rows x cols bf16 (leading dimension ld_src, any alignment)
// into dst with leading dimension ld_dst (a multiple of 8, >= cols; rows
// zero-padded), batch entries rows*ld_dst apart.
hipError_t launch_pack_rows(const uint16_t* src, int64_t ld_src, int64_t stride_src, uint16_t* dst, int64_t ld_dst,
                            int rows, int cols, int batch, hipStream_t st);

// Batch K x N bf16 matrices (leading dimension ld_src, batch stride s_src) into
// N x K (ld_dst >= K, a multiple of 8, dst 16-byte aligned; padding columns
// zeroed).  src_vec: source rows 16-byte aligned (128-bit loads).  Fails with
// hipErrorInvalidValue beyond 65535 batch entries or K tiles.
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t ld_src, int64_t s_src, uint16_t* dst, int64_t ld_dst,
                                 int64_t s_dst, int K, int N, int batch, bool src_vec, hipStream_t st);

// Calibration probes: MFMA rate on random operands (blocks x 4 waves, each
// 64*iters 32x32x16 MFMAs) and a streaming copy of `bytes` (multiple of 16).
hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st);
hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t st);
// Read-only streaming of `bytes` (multiple of 16); `out` holds blocks * 256 words.
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st);

// Calibration helpers: fill a buffer with pseudo-random bf16 in [-1, 1).
hipError_t launch_fill_random_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t st);

}  // namespace mkp
