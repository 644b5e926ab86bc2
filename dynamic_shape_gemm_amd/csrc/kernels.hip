// CDNA4 (gfx950) micro-kernel library.
//
// Every micro-kernel is one fixed uM x uN x uK tile; a workgroup runs one
// pipeline task: it walks its K range in uK steps, each step bringing the A
// (uM x uK) and B (uK x uN) tiles from HBM into LDS and running bf16 MFMAs on
// them with fp32 accumulation, then writes the fp32 tile back (MikPoly page,
// section 3 "micro-kernel performance model": load to local memory, compute
// with intermediates kept local, write back).  Start addresses, extents and
// K trip counts are run-time arguments (section 4, GPU platform).  Edge
// tiles never read or write outside the operands, so any shape is covered
// without padding them ("partial padding", section 3, polymerization
// strategy).
//
// Data path of one K step:
//   * Direct global->LDS loads (global_load_lds_dwordx4): each wave
//     instruction moves 64 x 16 bytes into 1 KB of LDS in lane order, with no
//     register staging.  S LDS stages keep S-1 steps in flight; a bare
//     barrier preceded by an explicit vmcnt wait releases exactly the step
//     about to be used (a full workgroup fence would drain every load).
//   * A is stored K-contiguous (as in HBM), rows 16-byte-chunk XOR swizzled.
//   * B is stored N-contiguous (as in HBM), rows 32-byte-segment XOR
//     swizzled, and read with the LDS transpose read (ds_read_b64_tr_b16),
//     which hands each lane four K-consecutive values of one B column.
//   * The MFMA (32x32x16 bf16, or 16x16x32 for 16-row wave tiles) takes the
//     B^T fragment first and the A^T fragment second, so each lane's results
//     come in runs of four consecutive columns of one C row (128-bit stores).
//   * A fallback path (register loads with zero fill) serves the last K step
//     when K is not a multiple of uK, operands whose rows are not 16-byte
//     aligned, and the last tile column when N is not a multiple of 8.
#include "kernels.h"

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

// The file builds as four translation units compiled side by side: part 1
// holds the single-tile kernels, the helper kernels and their launchers,
// parts 2 and 3 the two-tile kernels for B as K x N and as N x K, part 4 the
// convolution kernels; without MKP_PART it holds everything.
#ifndef MKP_PART
#define MKP_PART 0
#endif

#include <map>
#include <mutex>
#include <type_traits>

namespace mkp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_t;

// ---- fused epilogue -------------------------------------------------------

// Activations, branch-free on the native 2^x and reciprocal instructions.
//   sigmoid(z) = 1 / (1 + e^-z)
//   silu(x) = x sigmoid(x); the tanh form of GELU, x/2 (1 + tanh u), equals
//   x sigmoid(2u) since (1 + tanh u) / 2 = sigmoid(2u)
//   GELU, x Phi(x) = x/2 (1 + erf(x / sqrt 2)), with erf from Abramowitz &
//   Stegun, Handbook of Mathematical Functions, formula 7.1.26 (absolute
//   error <= 1.5e-7): for a >= 0, 1 - erf(a) = q(a) = P(t) e^{-a^2},
//   t = 1 / (1 + p a), P a degree-5 polynomial without constant term; so
//   1 + erf(x / sqrt 2) is q(|x| / sqrt 2) for x < 0 (no cancellation in the
//   negative tail) and 2 - q for x >= 0.
__device__ __forceinline__ float sigmoid_fast(float z) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

__device__ __forceinline__ float gelu_erf_fast(float x) {
    const float a = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * a);
    float poly = 1.061405429f;
    poly = fmaf(poly, t, -1.453152027f);
    poly = fmaf(poly, t, 1.421413741f);
    poly = fmaf(poly, t, -0.284496736f);
    poly = fmaf(poly, t, 0.254829592f);
    const float q = poly * t * __builtin_amdgcn_exp2f(-1.4426950408889634f * a * a);
    return 0.5f * x * (x < 0.0f ? q : 2.0f - q);
}

template <int ACT>
__device__ __forceinline__ float act_t(float v) {
    if constexpr (ACT == ACT_RELU) return v > 0.0f ? v : 0.0f;
    if constexpr (ACT == ACT_GELU) return gelu_erf_fast(v);
    if constexpr (ACT == ACT_GELU_TANH)
        return v * sigmoid_fast(2.0f * 0.79788456080286536f * (v + 0.044715f * v * v * v));
    if constexpr (ACT == ACT_SILU) return v * sigmoid_fast(v);
    return v;
}

__device__ __forceinline__ float act_apply(int act, float v) {
    switch (act) {
        case ACT_RELU: return act_t<ACT_RELU>(v);
        case ACT_GELU: return act_t<ACT_GELU>(v);
        case ACT_GELU_TANH: return act_t<ACT_GELU_TANH>(v);
        case ACT_SILU: return act_t<ACT_SILU>(v);
        default: return v;
    }
}

// bias[n..n+3] (zeros past nvalid, or without a bias)
__device__ __forceinline__ f32x4 load_bias4(const KEpi& e, int n, int nvalid) {
    f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if (e.bias != nullptr) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < nvalid) b[r] = e.bias[n + r];
    }
    return b;
}

// The output's current values at p[0..3] (zeros past nvalid); vec allows a
// 128-bit read.
__device__ __forceinline__ f32x4 read_old4(const float* p, bool vec, int nvalid) {
    f32x4 old = {0.0f, 0.0f, 0.0f, 0.0f};
    if (vec && nvalid >= 4) {
        old = *(const f32x4*)p;
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (r < nvalid) old[r] = p[r];
    }
    return old;
}

// Four consecutive values through the epilogue with the activation fixed at
// compile time (no beta term).
template <int ACT>
__device__ __forceinline__ f32x4 epi_apply4_t(float alpha, f32x4 b4, f32x4 v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = act_t<ACT>(fmaf(alpha, v[r], b4[r]));
    return v;
}

// Four consecutive values through the epilogue, given the old output values
// (used only when beta != 0) and the bias (load_bias4).
__device__ __forceinline__ f32x4 epi_apply4(const KEpi& e, f32x4 old, f32x4 b4, f32x4 v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float x = e.alpha * v[r];
        if (e.beta != 0.0f) x += e.beta * old[r];
        v[r] = act_apply(e.act, x + b4[r]);
    }
    return v;
}

// Four consecutive columns of one row at p (nvalid of them exist).
__device__ __forceinline__ f32x4 epi4(const KEpi& e, const float* p, bool vec, int nvalid, f32x4 b4, f32x4 v) {
    const f32x4 old = e.beta != 0.0f ? read_old4(p, vec, nvalid) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    return epi_apply4(e, old, b4, v);
}

__device__ __forceinline__ float epi1(const KEpi& e, const float* p, float bias, float v) {
    float x = e.alpha * v;
    if (e.beta != 0.0f) x += e.beta * *p;
    return act_apply(e.act, x + bias);
}

// A rows (uK*2 bytes) are XOR swizzled in 16-byte chunks: the 16 rows one
// fragment read touches land in 16 distinct 16-byte bank windows.
template <int BK>
__device__ __forceinline__ int swzA(int row);
template <>
__device__ __forceinline__ int swzA<64>(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// B rows (uN*2 bytes) are XOR swizzled in 32-byte segments so that one
// transposed read never hits a 32-byte bank window twice in a 32-lane pass.
// 16x16x32 fragments read 8 consecutive K rows of one segment; 32x32x16
// fragments read 4 consecutive K rows of two adjacent segments.
template <int BN, int MF>
__device__ __forceinline__ int swzB(int k) {
    if constexpr (MF == 16) return BN >= 128 ? (k & 7) : ((k >> 1) & 3);
    else return BN >= 128 ? ((k & 3) << 1) : (((k >> 1) & 1) << 1);
}

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int S_, bool PREREAD_ = false, bool BT_ = false,
          bool CONV_ = false>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, S = S_;
    static constexpr bool PREREAD = PREREAD_;   // read a whole stage's fragments before its MFMAs
    // B given as N x K (K-contiguous rows, the layout of a linear layer's
    // weights): its tile is stored like A's and read with the same 128-bit
    // fragment reads instead of the transposed ones
    static constexpr bool BT = BT_;
    // A gathered from an NHWC input (implicit-GEMM convolution, KArgs::conv)
    static constexpr bool CONV = CONV_;
    static_assert(!CONV || BT, "convolution kernels take the filters as an N x K matrix");
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = 64 * NW;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    // MFMA shape: 32x32x16 wherever the wave tile allows it (it reaches the
    // bf16 peak from one wave per SIMD), 16x16x32 for 16-row wave tiles
    static constexpr int MF = (WTM % 32 == 0 && WTN % 32 == 0) ? 32 : 16;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static constexpr int A_ROWB = BK * 2, B_ROWB = BT ? BK * 2 : BN * 2;
    static constexpr int A_BYTES = BM * A_ROWB, B_BYTES = BT ? BN * B_ROWB : BK * B_ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_SLOTS = A_BYTES / 16, B_SLOTS = B_BYTES / 16;
    static constexpr int A_GROUPS = A_SLOTS / 64, B_GROUPS = B_SLOTS / 64;   // 1 KB each
    static constexpr int A_IPW = (A_GROUPS + NW - 1) / NW, B_IPW = (B_GROUPS + NW - 1) / NW;
    static constexpr int IPS = A_IPW + B_IPW;        // LDS-DMA instructions per wave per step
    static constexpr bool JUNK = (A_GROUPS % NW) != 0 || (B_GROUPS % NW) != 0;
    static constexpr int LDS = S * STAGE + (JUNK ? 1024 : 0);
    static constexpr int A_RPT = (A_SLOTS + NT - 1) / NT, B_RPT = (B_SLOTS + NT - 1) / NT;
    // epilogue staging: one fragment row (MF rows x WTN columns) per wave,
    // rows padded by 4 floats to spread LDS banks where the stages leave room
    static constexpr int EPI_LD = (NW * MF * (WTN + 4) * 4 <= S * STAGE) ? WTN + 4 : WTN;
    static constexpr int EPI_WAVE_BYTES = MF * EPI_LD * 4;
    // the fused split-K reduction is compiled into all but the largest tile,
    // whose accumulators leave no registers for it
    static constexpr bool FUSED = BM * BN < 256 * 256;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BK == 64 || BK == 128, "uK must be 64 or 128");
    static_assert(BN >= 64 && BN % 64 == 0, "uN must be a multiple of 64");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "tiles must fill whole 1 KB groups");
    static_assert(S >= 2 && IPS * (S - 2) <= 63, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(NW * EPI_WAVE_BYTES <= S * STAGE, "epilogue staging fits in the stage buffers");
};

// LDS slot (16 bytes) -> (row, first element) of the A tile.
template <class T>
__device__ __forceinline__ void slotA(int p, int& row, int& col) {
    row = p / (T::BK / 8);
    col = ((p % (T::BK / 8)) ^ swzA<T::BK>(row)) * 8;
}
// LDS slot -> (k row, first column) of the B tile.
template <class T>
__device__ __forceinline__ void slotB(int p, int& k, int& col) {
    k = p / (T::BN / 8);
    const int pq = p % (T::BN / 8);
    col = ((((pq >> 1) ^ swzB<T::BN, T::MF>(k)) << 1) | (pq & 1)) * 8;
}

// LDS slot -> (row n, first K element) of a B tile stored N x K.
template <class T>
__device__ __forceinline__ void slotBt(int p, int& n, int& col) {
    n = p / (T::BK / 8);
    col = ((p % (T::BK / 8)) ^ swzA<T::BK>(n)) * 8;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Up to 8 consecutive bf16 values element by element (any alignment);
// missing elements read as zero; nothing is read when nvalid <= 0.
__device__ __forceinline__ u32x4 load8_elems(const uint16_t* p, int nvalid) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t lo = (2 * e < nvalid) ? (uint32_t)p[2 * e] : 0u;
        uint32_t hi = (2 * e + 1 < nvalid) ? (uint32_t)p[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// 8 consecutive bf16 values that are all inside the operand, from rows of
// any alignment: 4-byte words, shifted by 16 bits when the first value sits
// in the upper half of a word.  The words read never leave those holding
// the 8 values (so never a page beyond them).
__device__ __forceinline__ u32x4 load8_words(const uint16_t* p) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t* q = (const uint32_t*)(a & ~uintptr_t(3));
    if ((a & 2) == 0) return u32x4{q[0], q[1], q[2], q[3]};
    const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3], w4 = q[4];
    return u32x4{__builtin_amdgcn_alignbit(w1, w0, 16), __builtin_amdgcn_alignbit(w2, w1, 16),
                 __builtin_amdgcn_alignbit(w3, w2, 16), __builtin_amdgcn_alignbit(w4, w3, 16)};
}

// Up to 8 values: whole chunks by words, partial ones element by element.
__device__ __forceinline__ u32x4 load8_any(const uint16_t* p, int nvalid) {
    return nvalid >= 8 ? load8_words(p) : load8_elems(p, nvalid);
}

// Wait until at most N vector-memory operations of this wave are in flight
// and its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for the step about to be used while `ahead` later steps (each IPS
// direct-load instructions per wave, issued in order) stay in flight; the
// vmcnt immediate is chosen from the compile-time range 0 .. S-2.
template <class T, int A>
__device__ __forceinline__ void wait_upto(int ahead) {
    if constexpr (A <= 0) {
        wait_and_barrier<0>();
    } else {
        if (ahead >= A) {
            wait_and_barrier<A * T::IPS>();
            return;
        }
        wait_upto<T, A - 1>(ahead);
    }
}

template <class T>
__device__ __forceinline__ void wait_step(int ahead) {
    wait_upto<T, T::S - 2>(ahead);
}

// One direct global->LDS load: 16 bytes per lane, the wave's 64 chunks
// landing in lane order at `lds` (wave-uniform).  Written out here rather
// than through the compiler's builtin because the compiler's wait insertion
// cannot tell the stages of the one LDS array apart: before any fragment
// read it would wait for every direct load in flight -- including the ones
// just issued for later steps -- and the loads would never overlap the
// MFMAs.  The K loop's explicit waits (wait_step: a vmcnt count per step,
// then a barrier) order these loads with the reads instead.  Loads complete
// in issue order, so for the compiler's own loads an unseen direct load can
// only make its waits stricter.  M0 carries the LDS address (one wait state
// between writing it and the load that reads it).
// (M0 is reserved to the compiler, which sets it right before each of its
// own uses; the clobber still tells it this statement changes M0.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, lds_t* lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// Agent-coherent 16-byte accesses for the fused split-K exchange: sc1 makes
// a store write through the XCD's L2 to the level every XCD sees, and a load
// read from there rather than from a line its own L2 may hold (the memory
// model's encoding of agent-scope atomic loads and stores).  Their completion
// (vmcnt) is their visibility at agent scope, so the exchange needs no L2
// write-back or invalidate.  `base` is wave-uniform; byte offsets stay below
// 2^31.
constexpr int kCoherentAgent = 16;   // the sc1 cache-policy bit
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void store4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCoherentAgent);
}
__device__ __forceinline__ f32x4 load4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherentAgent));
}

// 16 bytes of C (or of a split-K partial) at element idx of base (wave-
// uniform), with the store policy of the launch: a streaming store (nt,
// KF_NT_C) or one written through to the level every XCD shares (sc1,
// KF_SC1_C) need not wait dirty in the XCD's L2 for the write-back at the
// kernel's end.  Both are buffer stores with those cache-policy bits (byte
// offsets below 2^31, which the host checks before it sets a flag); an
// ordinary store otherwise.  (A nontemporal global store in one branch and an
// ordinary one in the other would be merged into one ordinary store.)
constexpr int kStreaming = 2;   // the nt cache-policy bit
__device__ __forceinline__ int store_policy(int flags) {
    return ((flags & KF_NT_C) ? 1 : 0) | ((flags & KF_SC1_C) ? 2 : 0);
}
__device__ __forceinline__ void st4(float* base, int64_t idx, f32x4 v, int pol) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    if (pol == 1) __builtin_amdgcn_raw_buffer_store_b128(w, coherent_rsrc(base), (int)(idx * 4), 0, kStreaming);
    else if (pol == 2) __builtin_amdgcn_raw_buffer_store_b128(w, coherent_rsrc(base), (int)(idx * 4), 0, kCoherentAgent);
    else if (pol == 3)
        __builtin_amdgcn_raw_buffer_store_b128(w, coherent_rsrc(base), (int)(idx * 4), 0, kStreaming | kCoherentAgent);
    else *(f32x4*)(base + idx) = v;
}

struct TileCtx {
    const uint16_t* A;   // tile origin row m0 (row 0 of the tile), column 0; convolution: the input
    const uint16_t* B;   // tile origin column n0, row 0
    int64_t lda, ldb;
    int Mr, Nr;          // rows/columns of the tile inside the region
    int kend;            // end of this split's K range
    bool vecA, vecB;
    int row0;            // convolution: A row of the tile's row 0
    KConv cv;            // convolution geometry
};

// Convolution: offset of A(m, k) in the input, or -1 where it is padding.
[[maybe_unused]] __device__ __forceinline__ int64_t conv_offset(const KConv& v, int m, int k) {
    const int pq = v.P * v.Q;
    const int n = m / pq, pr = m - n * pq, p = pr / v.Q, q = pr - p * v.Q;
    const int rs = k / v.C, ch = k - rs * v.C, r = rs / v.S, s = rs - r * v.S;
    const int h = p * v.sh - v.ph + r * v.dh, w = q * v.sw - v.pw + s * v.dw;
    if ((unsigned)h >= (unsigned)v.H || (unsigned)w >= (unsigned)v.W) return -1;
    return (((int64_t)n * v.H + h) * v.W + w) * v.C + ch;
}

// Per-lane element offsets of the direct loads, fixed for a tile: rows and
// columns past the tile's valid extent are clamped to valid ones (they only
// feed C rows/columns that are never stored).  A step then adds a uniform
// base (A + k0, B + k0*ldb), so each load is a scalar base plus one 32-bit
// offset.
template <class T>
struct DmaOffsets {
    uint32_t a[T::A_IPW], b[T::B_IPW];
    // convolution: per A chunk, the input offset of its pixel's tap (0, 0)
    // plus the chunk's channel, and that tap's input row and column; the
    // current filter tap (r, s) and first channel c0 of the step, advanced
    // one step at a time (the direct-load steps come in order)
    int cbase[T::CONV ? T::A_IPW : 1];   // (32 bits: the host enables this path only when offsets fit)
    int ch0[T::CONV ? T::A_IPW : 1], cw0[T::CONV ? T::A_IPW : 1];
    int tr = 0, ts = 0, tc0 = 0;

    __device__ __forceinline__ void init(const TileCtx& c, int wave, int lane, int kbeg = 0) {
        if constexpr (T::CONV) {
            const int rs = kbeg / c.cv.C;
            tc0 = kbeg - rs * c.cv.C;
            tr = rs / c.cv.S;
            ts = rs - tr * c.cv.S;
        }
#pragma unroll
        for (int i = 0; i < T::A_IPW; ++i) {
            const int g = i * T::NW + wave;
            int row, col;
            slotA<T>(g * 64 + lane, row, col);
            row = min(row, c.Mr - 1);
            const bool real = (T::A_GROUPS % T::NW == 0) || g < T::A_GROUPS;
            if constexpr (T::CONV) {
                const KConv& v = c.cv;
                const int m = c.row0 + row, pq = v.P * v.Q;
                const int n = m / pq, pr = m - n * pq, p = pr / v.Q, q = pr - p * v.Q;
                ch0[i] = p * v.sh - v.ph;
                cw0[i] = q * v.sw - v.pw;
                cbase[i] = ((n * v.H + ch0[i]) * v.W + cw0[i]) * v.C + col;
                a[i] = 0u;
            } else {
                a[i] = real ? (uint32_t)(row * c.lda + col) : 0u;
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_IPW; ++i) {
            const int g = i * T::NW + wave;
            const bool real = (T::B_GROUPS % T::NW == 0) || g < T::B_GROUPS;
            if constexpr (T::BT) {
                int n, col;
                slotBt<T>(g * 64 + lane, n, col);
                n = min(n, c.Nr - 1);
                b[i] = real ? (uint32_t)(n * c.ldb + col) : 0u;
            } else {
                // chunks past the tile's last column repeat the last one
                // that holds a valid column; when N % 8 != 0 that chunk also
                // holds up to 7 columns past N, inside the same 16-byte block
                // as a valid one (so on a page the operand occupies), and they
                // feed only output columns >= N, which are never stored
                int k, col;
                slotB<T>(g * 64 + lane, k, col);
                col = min(col, (c.Nr - 1) & ~7);
                b[i] = real ? (uint32_t)(k * c.ldb + col) : 0u;
            }
        }
    }

    // Direct global->LDS loads of one full K step (convolution: the steps in
    // order, from the one init was given).
    __device__ __forceinline__ void issue(const TileCtx& c, int k0, lds_t* stage, lds_t* junk, int wave) {
        const uint16_t* ab = c.A + k0;
        const uint16_t* bb = T::BT ? c.B + k0 : c.B + (int64_t)k0 * c.ldb;
        if constexpr (T::CONV) {
            // the step's K columns are channels tc0.. of filter tap (tr, ts):
            // one uniform offset from each chunk's tap-(0, 0) position
            const KConv& v = c.cv;
            const int dr = tr * v.dh, ds = ts * v.dw;
            const int tap = (dr * v.W + ds) * v.C + tc0;
#pragma unroll
            for (int i = 0; i < T::A_IPW; ++i) {
                const int g = i * T::NW + wave;
                const bool real = (T::A_GROUPS % T::NW == 0) || g < T::A_GROUPS;
                const bool in = (unsigned)(ch0[i] + dr) < (unsigned)v.H && (unsigned)(cw0[i] + ds) < (unsigned)v.W;
                const uint16_t* src = in ? c.A + (int64_t)(cbase[i] + tap) : v.zero;
                dma16((const void*)src, real ? stage + g * 1024 : junk);
            }
            tc0 += T::BK;   // C is a multiple of uK on this path
            if (tc0 == v.C) {
                tc0 = 0;
                if (++ts == v.S) {
                    ts = 0;
                    ++tr;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < T::A_IPW; ++i) {
                const int g = i * T::NW + wave;
                const bool real = (T::A_GROUPS % T::NW == 0) || g < T::A_GROUPS;
                dma16((const void*)(ab + a[i]), real ? stage + g * 1024 : junk);
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_IPW; ++i) {
            const int g = i * T::NW + wave;
            const bool real = (T::B_GROUPS % T::NW == 0) || g < T::B_GROUPS;
            dma16((const void*)(bb + b[i]), real ? stage + T::A_BYTES + g * 1024 : junk);
        }
    }
};

// Register path of one K step: bounded, zero-filled loads, then LDS writes
// into the same swizzled layout the direct loads produce.  Slots move in
// batches of four per thread to bound register use.
template <class T>
__device__ __forceinline__ u32x4 reg_load_a(const TileCtx& c, int k0, int p) {
    int row, col;
    slotA<T>(p, row, col);
    const int k = k0 + col;
    if constexpr (T::CONV) {
        if (row >= c.Mr || k >= c.kend) return zero4();
        const int m = c.row0 + row;
        if (c.vecA) {
            // C % 8 == 0: the 8 columns are 8 channels of one tap, 16 aligned bytes
            const int64_t off = conv_offset(c.cv, m, k);
            return off < 0 ? zero4() : *(const u32x4*)(c.A + off);
        }
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t v2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int kk = k + 2 * e + h;
                const int64_t off = kk < c.kend ? conv_offset(c.cv, m, kk) : -1;
                v2[h] = off < 0 ? 0u : (uint32_t)c.A[off];
            }
            wd[e] = v2[0] | (v2[1] << 16);
        }
        return u32x4{wd[0], wd[1], wd[2], wd[3]};
    }
    if (row < c.Mr && k < c.kend) {
        const uint16_t* src = c.A + (int64_t)row * c.lda + k;
        return (c.vecA && k + 8 <= c.kend) ? *(const u32x4*)src : load8_any(src, c.kend - k);
    }
    return zero4();
}

template <class T>
__device__ __forceinline__ u32x4 reg_load_b(const TileCtx& c, int k0, int p) {
    if constexpr (T::BT) {
        int n, col;
        slotBt<T>(p, n, col);
        const int k = k0 + col;
        if (n < c.Nr && k < c.kend) {
            const uint16_t* src = c.B + (int64_t)n * c.ldb + k;
            // (the convolution tiles keep element loads: word loads push the
            // largest one's registers over the limit)
            if constexpr (T::CONV)
                return (c.vecB && k + 8 <= c.kend) ? *(const u32x4*)src : load8_elems(src, c.kend - k);
            return (c.vecB && k + 8 <= c.kend) ? *(const u32x4*)src : load8_any(src, c.kend - k);
        }
        return zero4();
    }
    int k, col;
    slotB<T>(p, k, col);
    const int kk = k0 + k;
    if (kk < c.kend && col < c.Nr) {
        const uint16_t* src = c.B + (int64_t)kk * c.ldb + col;
        return (c.vecB && col + 8 <= c.Nr) ? *(const u32x4*)src : load8_any(src, c.Nr - col);
    }
    return zero4();
}

template <class T>
__device__ __forceinline__ void reg_step(const TileCtx& c, int k0, lds_t* stage, int tid) {
    constexpr int TOT = T::A_SLOTS + T::B_SLOTS;
    for (int base = 0; base < TOT; base += 4 * T::NT) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = base + u * T::NT + tid;
            v[u] = p < T::A_SLOTS ? reg_load_a<T>(c, k0, p) : (p < TOT ? reg_load_b<T>(c, k0, p - T::A_SLOTS) : zero4());
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = base + u * T::NT + tid;
            if (p < TOT) *(u32x4 __attribute__((address_space(3)))*)(stage + p * 16) = v[u];
        }
    }
    // every load of this step has landed on every path (also where no lane
    // had an LDS write to make), so the compiler carries no pending load into
    // the K loop's fragment reads (vmcnt 0; the other counters left alone);
    // the convolution forms skip it (the largest one would spill)
    if constexpr (!T::CONV) __builtin_amdgcn_s_waitcnt(0x0F70);
}

// One LDS stage through 32x32x16 MFMAs.  Fragments are double-buffered in
// registers: the reads of K sub-step ks+1 are issued before the MFMAs of
// sub-step ks and interleaved with them, so LDS latency hides behind MFMA
// issue instead of stalling it.
template <class T>
__device__ __forceinline__ void read_frags32(const lds_t* sa, const lds_t* sb, int ks, int lane, int wm, int wn,
                                             bf16x8 (&xb)[T::FN], bf16x8 (&ya)[T::FM]) {
    // lane = 32h + 16cs + s16: K half h, column half cs
    const int h = lane >> 5, cs = (lane >> 4) & 1, s16 = lane & 15;
    const int kk = ks * 16;
    if constexpr (T::BT) {
        // N x K tile: the lane takes column n = lane & 31 of the block, K
        // columns 16ks + 8h .. +7 (the A fragments' K assignment)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int n = wn * T::WTN + j * 32 + (lane & 31);
            const int c1 = (kk >> 3) + h;
            xb[j] = __builtin_bit_cast(bf16x8, *(const u32x4 __attribute__((address_space(3)))*)(
                                                   sb + n * T::B_ROWB + ((c1 ^ swzA<T::BK>(n)) << 4)));
        }
    } else {
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int seg = ((wn * T::WTN + j * 32) >> 4) + cs;
            const int k1 = kk + 8 * h + (s16 >> 2), k2 = k1 + 4;
            const int o = (s16 & 3) * 8;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(
                sb + k1 * T::B_ROWB + ((seg ^ swzB<T::BN, 32>(k1)) << 5) + o));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(
                sb + k2 * T::B_ROWB + ((seg ^ swzB<T::BN, 32>(k2)) << 5) + o));
            xb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int row = wm * T::WTM + i * 32 + (lane & 31);
        const int c1 = (kk >> 3) + h;
        ya[i] = __builtin_bit_cast(bf16x8, *(const u32x4 __attribute__((address_space(3)))*)(
                                                sa + row * T::A_ROWB + ((c1 ^ swzA<T::BK>(row)) << 4)));
    }
}

template <class T, class Acc>
__device__ __forceinline__ void compute_stage32(const lds_t* sa, const lds_t* sb, Acc (&acc)[T::FM][T::FN], int lane,
                                                int wm, int wn) {
    constexpr int NKS = T::BK / 16;
    if constexpr (T::PREREAD) {
        // Every fragment of the stage is read up front into its own
        // registers; the scheduling fence keeps the compiler from sinking the
        // reads next to their MFMAs (which would expose LDS latency once per
        // sub-step), and the MFMAs then wait progressively.
        bf16x8 xb[NKS][T::FN], ya[NKS][T::FM];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) read_frags32<T>(sa, sb, ks, lane, wm, wn, xb[ks], ya[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[ks][j], ya[ks][i], acc[i][j], 0, 0, 0);
    } else {
        // Fragments double-buffered across sub-steps: the reads of ks+1 are
        // interleaved with the MFMAs of ks.
        constexpr int READS = 2 * T::FN + T::FM;
        constexpr int MFMAS = T::FM * T::FN;
        constexpr int PER = (READS + MFMAS - 1) / MFMAS;
        bf16x8 xb[2][T::FN], ya[2][T::FM];
        read_frags32<T>(sa, sb, 0, lane, wm, wn, xb[0], ya[0]);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < NKS) read_frags32<T>(sa, sb, ks + 1, lane, wm, wn, xb[cur ^ 1], ya[cur ^ 1]);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xb[cur][j], ya[cur][i], acc[i][j], 0, 0, 0);
            if (ks + 1 < NKS) {
#pragma unroll
                for (int t = 0; t < MFMAS; ++t) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (t * PER < READS) __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
                }
            }
        }
    }
}

// One LDS stage through 16x16x32 MFMAs (16-row wave tiles): per K sub-step
// of 32, each fragment is two 64-bit reads (N x K tiles and A), or two
// transposed reads (K x N tiles).
template <class T, class Acc>
__device__ __forceinline__ void compute_stage16(const lds_t* sa, const lds_t* sb, Acc (&acc)[T::FM][T::FN], int lane,
                                                int wm, int wn) {
    const int g4 = lane >> 4, s16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < T::BK / 32; ++ks) {
        const int kk = ks * 32;
        bf16x8 xb[T::FN], ya[T::FM];
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            if constexpr (T::BT) {
                // N x K tile: the A fragments' K assignment
                const int n = wn * T::WTN + j * 16 + s16;
                const int c1 = (kk >> 3) + (g4 >> 1), hb = (g4 & 1) * 8;
                const u32x2 lo = *(const u32x2 __attribute__((address_space(3)))*)(
                    sb + n * T::B_ROWB + ((c1 ^ swzA<T::BK>(n)) << 4) + hb);
                const u32x2 hi = *(const u32x2 __attribute__((address_space(3)))*)(
                    sb + n * T::B_ROWB + (((c1 + 2) ^ swzA<T::BK>(n)) << 4) + hb);
                xb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
                continue;
            }
            const int seg = (wn * T::WTN + j * 16) >> 4;
            const int k1 = kk + 4 * g4 + (s16 >> 2), k2 = k1 + 16;
            const int o = (s16 & 3) * 8;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(
                sb + k1 * T::B_ROWB + ((seg ^ swzB<T::BN, 16>(k1)) << 5) + o));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(
                sb + k2 * T::B_ROWB + ((seg ^ swzB<T::BN, 16>(k2)) << 5) + o));
            xb[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int row = wm * T::WTM + i * 16 + s16;
            const int c1 = (kk >> 3) + (g4 >> 1), hb = (g4 & 1) * 8;
            const u32x2 lo = *(const u32x2 __attribute__((address_space(3)))*)(
                sa + row * T::A_ROWB + ((c1 ^ swzA<T::BK>(row)) << 4) + hb);
            const u32x2 hi = *(const u32x2 __attribute__((address_space(3)))*)(
                sa + row * T::A_ROWB + (((c1 + 2) ^ swzA<T::BK>(row)) << 4) + hb);
            ya[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb[j], ya[i], acc[i][j], 0, 0, 0);
    }
}

// Map the flat workgroup id to (tile_m, tile_n, split, batch).  Workgroups
// are dealt round-robin to the 8 XCDs; ids are first regrouped so that each
// XCD receives a contiguous run of logical ids, then the logical id walks
// GROUP_M tile rows per tile column so neighbouring tiles on one XCD share
// A rows and B columns in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(int bid, int G, int tiles_m, int tiles_n, int splits, int& tm, int& tn,
                                         int& split, int& b) {
    const int q = G >> 3, r = G & 7;
    const int x = bid & 7;
    const int L = x * q + (x < r ? x : r) + (bid >> 3);
    const int T = tiles_m * tiles_n;
    const int tile = L % T;
    const int rest = L / T;
    split = rest % splits;
    b = rest / splits;
    const int per_group = GROUP_M * tiles_n;
    const int g = tile / per_group;
    const int first_m = g * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int in_g = tile % per_group;
    tm = first_m + in_g % gsz;
    tn = in_g / gsz;
}

// One pipeline task of tile T: workgroup `bid` of the `nblk` workgroups that
// serve the region described by args; smem is the workgroup's LDS (T::LDS
// bytes).
template <class T>
__device__ __forceinline__ void tile_task(KArgs args, int bid, int nblk, lds_t* smem) {
    lds_t* junk = smem + T::S * T::STAGE;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % T::WGM, wn = wave / T::WGM;

    int tm, tn, split, b;
    map_tile<8>(bid, nblk, args.tiles_m, args.tiles_n, args.splits, tm, tn, split, b);
    if (args.ngroups > 0) {
        // grouped call: switch to the B, N and C of the tile column's group
        // (constant indices only, so the argument block stays in registers)
        KGroup G = args.group[0];
#pragma unroll
        for (int i = 1; i < kMaxGroups; ++i)
            if (i < args.ngroups && tn >= args.group[i].tile0) G = args.group[i];
        tn -= G.tile0;
        args.B = G.B;
        args.ldb = G.ldb;
        args.N = G.N;
        args.flags = (args.flags & ~KF_VEC_B) | (G.flags & KF_VEC_B);
        if (args.splits == 1) {
            args.C = G.C;
            args.ldc = G.ldc;
            args.flags = (args.flags & ~(KF_VEC_C | KF_NT_C | KF_SC1_C)) | (G.flags & (KF_VEC_C | KF_NT_C));
        } else {
            args.C += (int64_t)G.tile0 * T::BN;   // the group's workspace columns
        }
        args.counters = nullptr;
    }
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    TileCtx c;
    if constexpr (T::CONV) {
        c.A = args.A;   // the input; rows are gathered
        c.row0 = args.conv.m0 + m0;
        c.cv = args.conv;
    } else {
        c.A = args.A + (int64_t)b * args.sA + (int64_t)m0 * args.lda;
    }
    // B tile origin: column n0 of a K x N matrix, or row n0 of an N x K one
    c.B = args.B + (int64_t)b * args.sB + (T::BT ? (int64_t)n0 * args.ldb : (int64_t)n0);
    c.lda = args.lda;
    c.ldb = args.ldb;
    c.Mr = args.M - m0;
    c.Nr = args.N - n0;
    const int kbeg = split * args.steps_per_split * T::BK;
    c.kend = min(args.K, kbeg + args.steps_per_split * T::BK);
    c.vecA = args.flags & KF_VEC_A;
    c.vecB = args.flags & KF_VEC_B;
    const int nsteps = (c.kend - kbeg + T::BK - 1) / T::BK;
    // direct loads need 16-byte aligned rows and 32-bit tile offsets (host
    // clears the vector flags for leading dimensions too large for them)
    const bool dma_tile = c.vecA && c.vecB && (!T::CONV || (args.flags & KF_CONV_DMA));
    const int dma_steps = dma_tile ? (c.kend - kbeg) / T::BK : 0;   // full steps

    DmaOffsets<T> dma;
    if (dma_tile) dma.init(c, wave, lane, kbeg);
    auto load_step = [&](int s) {
        lds_t* st = smem + (s % T::S) * T::STAGE;
        const int k0 = kbeg + s * T::BK;
        if (s < dma_steps) dma.issue(c, k0, st, junk, wave);
        else reg_step<T>(c, k0, st, tid);
    };

    using acc_t = typename std::conditional<T::MF == 32, f32x16, f32x4>::type;
    acc_t acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = acc_t{};

#pragma unroll
    for (int s = 0; s < T::S - 1; ++s)
        if (s < nsteps) load_step(s);

    const int g4 = lane >> 4, s16 = lane & 15;
    for (int s = 0; s < nsteps; ++s) {
        wait_step<T>(min(T::S - 2, nsteps - 1 - s));
        if (s + T::S - 1 < nsteps) load_step(s + T::S - 1);
        const lds_t* sa = smem + (s % T::S) * T::STAGE;
        const lds_t* sb = sa + T::A_BYTES;
        if constexpr (T::MF == 32) {
            compute_stage32<T>(sa, sb, acc, lane, wm, wn);
        } else {
            compute_stage16<T>(sa, sb, acc, lane, wm, wn);
        }
    }

    // Epilogue: every lane holds runs of four consecutive columns of one C row.
    float* __restrict__ C = args.C + (int64_t)b * args.sC + (int64_t)split * args.sCsplit +
                            (int64_t)m0 * args.ldc + n0;
    const bool vecC = args.flags & KF_VEC_C;
    const int ntC = store_policy(args.flags);
    auto store4 = [&](float* base, int64_t ld, bool vec, int m, int n, f32x4 v) {
        if (m >= c.Mr) return;
        float* p = base + (int64_t)m * ld + n;
        if (vec && n + 4 <= c.Nr) {
            st4(base, (int64_t)m * ld + n, v, ntC);
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < c.Nr) p[r] = v[r];
        }
    };
    // final values go through the fused epilogue (one split, or the fused
    // reduction's sum; two-pass split-K leaves it to the reduction)
    const bool epi = args.flags & KF_EPI;
    auto emit4 = [&](float* base, int64_t ld, bool vec, int m, int n, f32x4 v) {
        if (m >= c.Mr) return;
        if (epi) v = epi4(args.epi, base + (int64_t)m * ld + n, vec, c.Nr - n, load_bias4(args.epi, n0 + n, c.Nr - n), v);
        store4(base, ld, vec, m, n, v);
    };
    // Plain epilogue: the tile goes through LDS one fragment row at a time
    // so that every store instruction writes contiguous row segments.
    const bool epi_here = epi && args.splits == 1;
    // this split's partial goes to the fused reduction (workspace rows are
    // 16-byte aligned, so the vector store loop writes it)
    const bool fused_split = T::FUSED && args.splits > 1 && args.counters != nullptr;
    const int col0 = wn * T::WTN;   // first tile column of this wave
    constexpr int C4 = T::WTN / 4;  // 16-byte chunks per staged row
    static_assert(64 % C4 == 0, "a lane's chunk column must not change across the store loop");
    // 16-byte stores on unaligned rows (below) everywhere but in the
    // convolution form of the largest tile, whose registers they would spill
    constexpr bool kWideUnaligned = !(T::CONV && T::BM * T::BN >= 256 * 256);
    // with the epilogue, each lane's bias chunk is loaded once: its column is
    // the same in every row it stores
    f32x4 bias4 = {0.0f, 0.0f, 0.0f, 0.0f};
    float bias1[(T::WTN + 63) / 64] = {};
    if (epi_here) {
        const int cl = col0 + (lane % C4) * 4;
        bias4 = load_bias4(args.epi, n0 + cl, c.Nr - cl);
#pragma unroll
        for (int c0 = 0; c0 < T::WTN; c0 += 64)
            bias1[c0 / 64] = (args.epi.bias != nullptr && col0 + c0 + lane < c.Nr) ? args.epi.bias[n0 + col0 + c0 + lane]
                                                                                  : 0.0f;
    }
    __syncthreads();   // every wave is done with the K-loop stages
    float __attribute__((address_space(3)))* stg =
        (float __attribute__((address_space(3)))*)(smem + wave * T::EPI_WAVE_BYTES);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        // fragment row i of this wave: MF rows x WTN columns, rows padded by 4 floats
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            if constexpr (T::MF == 32) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = lane & 31, col = j * 32 + 8 * q + 4 * (lane >> 5);
                    *(f32x4 __attribute__((address_space(3)))*)(stg + r * T::EPI_LD + col) =
                        f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                }
            } else {
                *(f32x4 __attribute__((address_space(3)))*)(stg + s16 * T::EPI_LD + j * 16 + g4 * 4) = acc[i][j];
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's LDS writes land before its reads
        const int row0 = wm * T::WTM + i * T::MF;             // tile row of staged row 0
        constexpr int ITS = (T::MF * C4 + 63) / 64;
        if (vecC && epi_here && args.epi.beta == 0.0f) {
            // no reads in this loop (a load would make the compiler wait for
            // every earlier store, vmcnt counting both, before its use), and
            // the activation chosen once, outside it
            const int n = col0 + (lane % C4) * 4;
            auto rows = [&](auto act_tag) {
                constexpr int ACT = decltype(act_tag)::value;
#pragma unroll 1
                for (int it = 0; it < ITS; ++it) {
                    const int id = it * 64 + lane;
                    if ((T::MF * C4) % 64 == 0 || id < T::MF * C4) {
                        const int r = id / C4;
                        const f32x4 v =
                            *(const f32x4 __attribute__((address_space(3)))*)(stg + r * T::EPI_LD + (n - col0));
                        if (row0 + r < c.Mr)
                            store4(C, args.ldc, true, row0 + r, n, epi_apply4_t<ACT>(args.epi.alpha, bias4, v));
                    }
                }
            };
            switch (args.epi.act) {
                case ACT_RELU: rows(std::integral_constant<int, ACT_RELU>{}); break;
                case ACT_GELU: rows(std::integral_constant<int, ACT_GELU>{}); break;
                case ACT_GELU_TANH: rows(std::integral_constant<int, ACT_GELU_TANH>{}); break;
                case ACT_SILU: rows(std::integral_constant<int, ACT_SILU>{}); break;
                default: rows(std::integral_constant<int, ACT_NONE>{}); break;
            }
        } else if (vecC && epi_here) {
            // the lane's column n is fixed; the old values of the next row
            // are read one iteration ahead
            const int n = col0 + (lane % C4) * 4;
            const bool rd = true;
            auto old_at = [&](int it) -> f32x4 {
                const int id = it * 64 + lane;
                const int m = row0 + id / C4;
                if (!rd || it >= ITS || ((T::MF * C4) % 64 != 0 && id >= T::MF * C4) || m >= c.Mr)
                    return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                return read_old4(C + (int64_t)m * args.ldc + n, true, c.Nr - n);
            };
            f32x4 old_next = old_at(0);
#pragma unroll 1
            for (int it = 0; it < ITS; ++it) {
                const f32x4 old = old_next;
                old_next = old_at(it + 1);
                const int id = it * 64 + lane;
                if ((T::MF * C4) % 64 == 0 || id < T::MF * C4) {
                    const int r = id / C4;
                    if (row0 + r < c.Mr) {
                        f32x4 v = *(const f32x4 __attribute__((address_space(3)))*)(stg + r * T::EPI_LD + (n - col0));
                        store4(C, args.ldc, true, row0 + r, n, epi_apply4(args.epi, old, bias4, v));
                    }
                }
            }
        } else if (vecC && fused_split) {
            // a split's partial tile for the fused reduction: written
            // through to where the last-arriving split, on any XCD, reads it
            const __amdgpu_buffer_rsrc_t rc = coherent_rsrc(C);
#pragma unroll 1
            for (int it = 0; it < ITS; ++it) {
                const int id = it * 64 + lane;
                if ((T::MF * C4) % 64 == 0 || id < T::MF * C4) {
                    const int r = id / C4, c4 = (id % C4) * 4;
                    const f32x4 v = *(const f32x4 __attribute__((address_space(3)))*)(stg + r * T::EPI_LD + c4);
                    // whole chunks up to the row's last column (workspace
                    // rows are padded to a multiple of 4 floats)
                    if (row0 + r < c.Mr && col0 + c4 < c.Nr)
                        store4_coherent(rc, (uint32_t)(((row0 + r) * args.ldc + col0 + c4) * 4), v);
                }
            }
        } else if (vecC) {
#pragma unroll 1
            for (int it = 0; it < ITS; ++it) {
                const int id = it * 64 + lane;
                if ((T::MF * C4) % 64 == 0 || id < T::MF * C4) {
                    const int r = id / C4, c4 = (id % C4) * 4;
                    const f32x4 v = *(const f32x4 __attribute__((address_space(3)))*)(stg + r * T::EPI_LD + c4);
                    store4(C, args.ldc, true, row0 + r, col0 + c4, v);
                }
            }
        } else if (kWideUnaligned && !epi_here) {
            // Unaligned rows (4-byte aligned only): each row's segment of
            // this wave's columns is written with 16-byte stores from its
            // first 16-byte boundary on, 4 columns per lane as in the
            // aligned loop; the at most three columns before that boundary
            // and three after the last whole chunk go out one by one below.
            const int W = min(T::WTN, c.Nr - col0);   // valid columns of the strip
            if (W > 0) {
#pragma unroll 1
                for (int it = 0; it < ITS; ++it) {
                    const int id = it * 64 + lane;
                    if ((T::MF * C4) % 64 == 0 || id < T::MF * C4) {
                        const int r = id / C4, j = id % C4;
                        const int m = row0 + r;
                        float* d = C + (int64_t)m * args.ldc + col0;
                        const int h = min((int)((0u - (uint32_t)(uintptr_t)d) >> 2) & 3, W);
                        const int col = h + 4 * j;
                        if (m < c.Mr && col + 4 <= W) {
                            const float __attribute__((address_space(3)))* sr = stg + r * T::EPI_LD + col;
                            st4(C, (int64_t)m * args.ldc + col0 + col, f32x4{sr[0], sr[1], sr[2], sr[3]}, ntC);
                        }
                    }
                }
#pragma unroll 1
                for (int r0 = 0; r0 < T::MF; r0 += 8) {
                    const int r = r0 + (lane >> 3), e = lane & 7;
                    const int m = row0 + r;
                    float* d = C + (int64_t)m * args.ldc + col0;
                    const int h = min((int)((0u - (uint32_t)(uintptr_t)d) >> 2) & 3, W);
                    const int t0 = h + ((W - h) & ~3);   // first column after the whole chunks
                    const int col = e < h ? e : t0 + (e - h);
                    if (m < c.Mr && (e < h || col < W)) d[col] = stg[r * T::EPI_LD + col];
                }
            }
        } else {
            // unaligned rows with the epilogue: lanes walk one row's
            // columns, one float each
#pragma unroll 1
            for (int r = 0; r < T::MF; ++r) {
                const int m = row0 + r;
                if (m >= c.Mr) break;
                float* dst = C + (int64_t)m * args.ldc + col0;
#pragma unroll
                for (int c0 = 0; c0 < T::WTN; c0 += 64) {
                    const int col = c0 + lane;
                    if ((T::WTN % 64 == 0 || col < T::WTN) && col0 + col < c.Nr) {
                        const float v = stg[r * T::EPI_LD + col];
                        dst[col] = epi_here ? epi1(args.epi, dst + col, bias1[c0 / 64], v) : v;
                    }
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next row overwrites
    }
    if (fused_split) {
        // Fused split-K reduction.  Every split has written its partial tile
        // through to the level all XCDs share (the rows above, into the
        // workspace).  Once every wave's stores have completed -- and so
        // are visible there -- wave 0 counts the arrival with an
        // agent-scope atomic.  The last split to arrive reads all partials
        // with agent-coherent loads (not from its own L2, which may hold
        // stale lines of the workspace) and sums them in split order -- the
        // same order whichever split arrives last -- whole rows at a time
        // (16 bytes per lane, consecutive lanes along a row), then writes C
        // through the epilogue.  No L2 write-back or invalidate is needed.
        // The arrival flag lives in the stage memory, idle after the
        // epilogue (every wave is past its staging once the barrier is passed).
        int __attribute__((address_space(3)))* s_last_p = (int __attribute__((address_space(3)))*)smem;
        __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have completed
        __syncthreads();
        int* cnt = args.counters + (int64_t)b * args.tiles_m * args.tiles_n + tm * args.tiles_n + tn;
        if (wave == 0) {
            int last = 0;
            if (lane == 0)
                last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == args.splits - 1;
            last = __builtin_amdgcn_readfirstlane(last);
            if (lane == 0) *s_last_p = last;
        }
        __syncthreads();
        if (!*s_last_p) return;
        const float* Wt = args.C + (int64_t)b * args.sC + (int64_t)m0 * args.ldc + n0;   // split 0's tile
        float* Co = args.Cout + (int64_t)b * args.sCout + (int64_t)m0 * args.ldcout + n0;
        const bool vecCo = args.flags & KF_VEC_COUT;
        const int rows = min(c.Mr, T::BM);
        constexpr int CH = T::BN / 4;   // 16-byte chunks per tile row
#pragma unroll 1
        for (int id = tid; id < rows * CH; id += T::NT) {
            const int m = id / CH, n = (id % CH) * 4;
            if (n >= c.Nr) continue;
            const uint32_t e = (uint32_t)((m * args.ldc + n) * 4);   // workspace rows: 16-byte aligned
            // partials in split order, eight loads issued before their adds
            // (one load per add would wait out a round trip per split)
            f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int z0 = 0; z0 < args.splits; z0 += 8) {
                f32x4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (z0 + u < args.splits) v[u] = load4_coherent(coherent_rsrc(Wt + (int64_t)(z0 + u) * args.sCsplit), e);
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (z0 + u < args.splits) sum = (z0 + u == 0) ? v[u] : sum + v[u];
            }
            emit4(Co, args.ldcout, vecCo, m, n, sum);
        }
        if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Every library launch goes through here: with the thread's launch-timing
// slot set, the kernel's own start and end go into its events.
template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t st, Args... args) {
    LaunchEvents& ev = launch_events();
    if (ev.start != nullptr) {
        const LaunchEvents use = ev;
        ev = LaunchEvents{};
        hipExtLaunchKernelGGL(kernel, grid, block, 0, st, use.start, use.stop, 0, args...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
    }
    return hipGetLastError();
}

template <class T>
__global__ __launch_bounds__(T::NT) void gemm_tile_kernel(KArgs args) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[T::LDS];
    tile_task<T>(args, blockIdx.x, gridDim.x, (lds_t*)smem_raw);
}

template <class T>
hipError_t launch_tile(const KArgs& a, dim3 grid, hipStream_t st) {
    return launch_kernel(gemm_tile_kernel<T>, grid, dim3(T::NT), st, a);
}

// ---- skinny-M tiles: the K range split across the waves ---------------------
//
// For outputs with few rows the tile count of a plain tile is too small to
// fill the CUs, and splitting K across workgroups costs a second pass over
// fp32 partials.  Here the KW waves of one workgroup split K instead: wave w
// takes the 64-wide K chunks w, w + KW, w + 2 KW, ... of the workgroup's K
// range, each through its own S-stage LDS pipeline (direct loads, no
// barrier: a wave waits only for its own loads), so one K step of the tile
// is 64 KW deep.  Every wave accumulates the whole BM x BN tile; at the end
// the waves' sums meet in LDS (added in wave order) and go out as C -- or
// as one split's partial when the plan also splits K across workgroups.
template <int BM_, int BN_, int KW_, int S_, bool BT_>
struct WSplit {
    static constexpr int BM = BM_, BN = BN_, KW = KW_, S = S_;
    static constexpr bool BT = BT_;
    static constexpr int NT = 64 * KW;
    static constexpr int BK = 64 * KW;                       // K per step of the workgroup (the table's uK)
    using T1 = Tile<BM, BN, 64, 1, 1, S, false, BT>;        // one wave's pipeline over 64-wide chunks
    static constexpr int WAVE_LDS = S * T1::STAGE;
    static constexpr int RED_LD = BN + 4;                    // staged row, padded by 4 floats
    static constexpr int RED = KW * BM * RED_LD * 4;
    static constexpr int LDS = (KW * WAVE_LDS > RED ? KW * WAVE_LDS : RED);
    static_assert(!T1::JUNK, "a wave's chunk must fill whole 1 KB load groups");
    static_assert(T1::IPS * (S - 1) <= 63, "vmcnt range");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Wait until at most A chunks' direct loads of this wave are in flight and
// its LDS reads are done (no barrier: the stages are the wave's own).
template <class T1, int A>
__device__ __forceinline__ void wave_wait_upto(int ahead) {
    if constexpr (A <= 0) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    } else {
        if (ahead >= A) {
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(A * T1::IPS) : "memory");
            return;
        }
        wave_wait_upto<T1, A - 1>(ahead);
    }
}

template <class W>
__device__ __forceinline__ void wsplit_task(KArgs args, int bid, int nblk, lds_t* smem) {
    using T1 = typename W::T1;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    int tm, tn, split, b;
    map_tile<8>(bid, nblk, args.tiles_m, args.tiles_n, args.splits, tm, tn, split, b);
    if (args.ngroups > 0) {
        // grouped call: the tile column's group (as in tile_task)
        KGroup G = args.group[0];
#pragma unroll
        for (int i = 1; i < kMaxGroups; ++i)
            if (i < args.ngroups && tn >= args.group[i].tile0) G = args.group[i];
        tn -= G.tile0;
        args.B = G.B;
        args.ldb = G.ldb;
        args.N = G.N;
        args.flags = (args.flags & ~KF_VEC_B) | (G.flags & KF_VEC_B);
        if (args.splits == 1) {
            args.C = G.C;
            args.ldc = G.ldc;
            args.flags = (args.flags & ~(KF_VEC_C | KF_NT_C | KF_SC1_C)) | (G.flags & (KF_VEC_C | KF_NT_C));
        } else {
            args.C += (int64_t)G.tile0 * W::BN;
        }
        args.counters = nullptr;
    }
    const int m0 = tm * W::BM, n0 = tn * W::BN;
    TileCtx c;
    c.A = args.A + (int64_t)b * args.sA + (int64_t)m0 * args.lda;
    c.B = args.B + (int64_t)b * args.sB + (W::BT ? (int64_t)n0 * args.ldb : (int64_t)n0);
    c.lda = args.lda;
    c.ldb = args.ldb;
    c.Mr = args.M - m0;
    c.Nr = args.N - n0;
    const int kbeg = split * args.steps_per_split * W::BK;
    c.kend = min(args.K, kbeg + args.steps_per_split * W::BK);
    c.vecA = args.flags & KF_VEC_A;
    c.vecB = args.flags & KF_VEC_B;
    const int nchunks = (c.kend - kbeg + 63) / 64;
    const bool dma_tile = c.vecA && c.vecB;
    const int dma_chunks = dma_tile ? (c.kend - kbeg) / 64 : 0;   // full chunks
    const int mine = nchunks > wave ? (nchunks - wave + W::KW - 1) / W::KW : 0;

    lds_t* ws = smem + wave * W::WAVE_LDS;
    DmaOffsets<T1> dma;
    if (dma_tile) dma.init(c, 0, lane);
    auto load = [&](int j) {   // this wave's j-th chunk
        const int q = wave + j * W::KW;
        lds_t* st = ws + (j % W::S) * T1::STAGE;
        const int k0 = kbeg + q * 64;
        if (q < dma_chunks) dma.issue(c, k0, st, st, 0);
        else reg_step<T1>(c, k0, st, lane);
    };

    using acc_t = typename std::conditional<T1::MF == 32, f32x16, f32x4>::type;
    acc_t acc[T1::FM][T1::FN];
#pragma unroll
    for (int i = 0; i < T1::FM; ++i)
#pragma unroll
        for (int j = 0; j < T1::FN; ++j) acc[i][j] = acc_t{};

#pragma unroll
    for (int j = 0; j < W::S - 1; ++j)
        if (j < mine) load(j);
    // chunk j+S-1 goes into the stage of chunk j-1 (whose reads have
    // completed) before the wait for chunk j, so S chunks are in flight
    // across the wait
    for (int j = 0; j < mine; ++j) {
        if (j + W::S - 1 < mine) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            load(j + W::S - 1);
        }
        wave_wait_upto<T1, W::S - 1>(min(W::S - 1, mine - 1 - j));
        const lds_t* sa = ws + (j % W::S) * T1::STAGE;
        const lds_t* sb = sa + T1::A_BYTES;
        if constexpr (T1::MF == 32) compute_stage32<T1>(sa, sb, acc, lane, 0, 0);
        else compute_stage16<T1>(sa, sb, acc, lane, 0, 0);
    }

    // the waves' sums meet in LDS: wave w's tile at rows of RED_LD floats
    __syncthreads();   // every wave is done with its stages
    float __attribute__((address_space(3)))* red = (float __attribute__((address_space(3)))*)smem;
    float __attribute__((address_space(3)))* mine_t = red + wave * W::BM * W::RED_LD;
#pragma unroll
    for (int i = 0; i < T1::FM; ++i)
#pragma unroll
        for (int j = 0; j < T1::FN; ++j) {
            if constexpr (T1::MF == 32) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = i * 32 + (lane & 31), col = j * 32 + 8 * q + 4 * (lane >> 5);
                    *(f32x4 __attribute__((address_space(3)))*)(mine_t + r * W::RED_LD + col) =
                        f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                }
            } else {
                const int r = i * 16 + (lane & 15), col = j * 16 + (lane >> 4) * 4;
                *(f32x4 __attribute__((address_space(3)))*)(mine_t + r * W::RED_LD + col) = acc[i][j];
            }
        }
    __syncthreads();

    // sum in wave order, 16 bytes per thread along the rows, and store
    float* C = args.C + (int64_t)b * args.sC + (int64_t)split * args.sCsplit + (int64_t)m0 * args.ldc + n0;
    const bool vecC = args.flags & KF_VEC_C;
    const bool epi = (args.flags & KF_EPI) && args.splits == 1;
    constexpr int CH = W::BN / 4;
    const int rows = min(c.Mr, W::BM);
#pragma unroll 1
    for (int id = tid; id < rows * CH; id += W::NT) {
        const int m = id / CH, n = (id % CH) * 4;
        if (n >= c.Nr) continue;
        f32x4 v = *(const f32x4 __attribute__((address_space(3)))*)(red + m * W::RED_LD + n);
#pragma unroll
        for (int w = 1; w < W::KW; ++w)
            v += *(const f32x4 __attribute__((address_space(3)))*)(red + (w * W::BM + m) * W::RED_LD + n);
        float* p = C + (int64_t)m * args.ldc + n;
        if (epi) v = epi4(args.epi, p, vecC, c.Nr - n, load_bias4(args.epi, n0 + n, c.Nr - n), v);
        if (vecC && n + 4 <= c.Nr) {
            st4(C, (int64_t)m * args.ldc + n, v, store_policy(args.flags));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < c.Nr) p[r] = v[r];
        }
    }
}

template <class W>
__global__ __launch_bounds__(W::NT) void gemm_wsplit_kernel(KArgs args) {
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[W::LDS];
    wsplit_task<W>(args, blockIdx.x, gridDim.x, (lds_t*)smem_raw);
}

template <class W>
hipError_t launch_wsplit(const KArgs& a, dim3 grid, hipStream_t st) {
    return launch_kernel(gemm_wsplit_kernel<W>, grid, dim3(W::NT), st, a);
}


// The two regions of a plan in one launch: workgroups [0, n1) run tile T1
// over region a1, the others tile T2 over region a2.  The hardware hands out
// workgroups in order, so the second region's tiles start as soon as slots
// free up in the first region's last wave (the merged-wave view of the
// MikPoly page's case study).  Both tiles use the same workgroup size, and
// the LDS of the larger one leaves the number of resident workgroups per CU
// of each unchanged.
template <class T1, class T2>
__global__ __launch_bounds__(T1::NT) void gemm_dual_kernel(KArgs a1, KArgs a2, int n1) {
    static_assert(T1::NT == T2::NT, "both tiles must use the same workgroup size");
    constexpr int L = T1::LDS > T2::LDS ? T1::LDS : T2::LDS;
    constexpr int kLdsPerCu = 160 * 1024;
    static_assert(kLdsPerCu / (L + 16) >= (kLdsPerCu / (T1::LDS + 16) < kLdsPerCu / (T2::LDS + 16)
                                              ? kLdsPerCu / (T1::LDS + 16)
                                              : kLdsPerCu / (T2::LDS + 16)),
                  "pairing must not lower the resident workgroups per CU");
    __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[L];
    if ((int)blockIdx.x < n1) tile_task<T1>(a1, blockIdx.x, n1, (lds_t*)smem_raw);
    else tile_task<T2>(a2, (int)blockIdx.x - n1, (int)gridDim.x - n1, (lds_t*)smem_raw);
}

template <class T1, class T2>
hipError_t launch_dual(const KArgs& a1, const KArgs& a2, int n1, dim3 grid, hipStream_t st) {
    return launch_kernel(gemm_dual_kernel<T1, T2>, grid, dim3(T1::NT), st, a1, a2, n1);
}

#if MKP_PART == 0 || MKP_PART == 1
template <bool EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ W, int splits, int64_t sWs,
                                                            int64_t sWb, int64_t ldw, float* __restrict__ C,
                                                            int64_t ldc, int64_t sC, int M, int N, int batch,
                                                            int vec, KEpi epi) {
    const int nq = (N + 3) >> 2;
    const int64_t per = (int64_t)M * nq;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per * batch) return;
    const int b = (int)(idx / per);
    const int64_t e = idx % per;
    const int m = (int)(e / nq);
    const int n = (int)(e % nq) * 4;
    f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    if (splits > 0) {
        // partials in split order; eight loads are issued before the first
        // add (a load per iteration would wait out one memory round trip
        // per split)
        const float* w = W + (int64_t)b * sWb + (int64_t)m * ldw + n;
        s = *(const f32x4*)w;
        for (int z0 = 1; z0 < splits; z0 += 8) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (z0 + u < splits) v[u] = *(const f32x4*)(w + (int64_t)(z0 + u) * sWs);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (z0 + u < splits) s += v[u];
        }
    }
    float* p = C + (int64_t)b * sC + (int64_t)m * ldc + n;
    if (EPI) s = epi4(epi, p, vec & 1, N - n, load_bias4(epi, n, N - n), s);
    if ((vec & 1) && n + 4 <= N) {
        st4(C, (int64_t)b * sC + (int64_t)m * ldc + n, s, (vec & 2) ? 1 : 0);
    } else {
        for (int r = 0; r < 4; ++r)
            if (n + r < N) p[r] = s[r];
    }
}

// Copy rows of bf16 into a staging buffer whose rows start 16-byte aligned
// (leading dimension a multiple of 8 elements), zero-padding each row up to
// it: operands with unaligned rows then take the direct-load path.  Each
// thread writes one 16-byte chunk; reads are element-wise (any alignment).
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                        int64_t stride_src, uint16_t* __restrict__ dst,
                                                        int64_t ld_dst, int rows, int cols, int batch) {
    const int64_t chunks_per_row = ld_dst >> 3;
    const int64_t per = (int64_t)rows * chunks_per_row;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per * batch) return;
    const int b = (int)(idx / per);
    const int64_t e = idx % per;
    const int r = (int)(e / chunks_per_row);
    const int c = (int)(e % chunks_per_row) * 8;
    const uint16_t* s = src + (int64_t)b * stride_src + (int64_t)r * ld_src + c;
    *(u32x4*)(dst + (int64_t)b * rows * ld_dst + (int64_t)r * ld_dst + c) = load8_elems(s, cols - c);
}

// dst[b][n][k] = src[b][k][n] for a K x N bf16 matrix (leading dimension
// ld_src) into N x K (leading dimension ld_dst >= K, a multiple of 8, rows
// 16-byte aligned; columns K..ld_dst-1 are zeroed).  One 64 x 64 tile per
// workgroup through LDS: 16-byte loads along the rows of the source (element
// loads when its rows are not 16-byte aligned) and 16-byte stores along the
// rows of the target.
template <bool VEC>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                             int64_t s_src, uint16_t* __restrict__ dst,
                                                             int64_t ld_dst, int64_t s_dst, int K, int N) {
    __shared__ __attribute__((aligned(16))) uint16_t t[64][72];   // [k][n], rows of 144 bytes
    const int tid = threadIdx.x;
    const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
    const uint16_t* sb = src + (int64_t)blockIdx.z * s_src;
    uint16_t* db = dst + (int64_t)blockIdx.z * s_dst;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = it * 256 + tid, r = q >> 3, c8 = (q & 7) * 8;
        const int k = k0 + r, n = n0 + c8;
        u32x4 v = zero4();
        if (k < K) {
            const uint16_t* p = sb + (int64_t)k * ld_src + n;
            v = (VEC && n + 8 <= N) ? *(const u32x4*)p : load8_elems(p, N - n);
        }
        *(u32x4*)&t[r][c8] = v;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = it * 256 + tid, r = q >> 3, c8 = (q & 7) * 8;
        const int n = n0 + r, k = k0 + c8;
        if (n >= N || k >= ld_dst) continue;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = k + 2 * e < K ? t[c8 + 2 * e][r] : 0u;
            const uint32_t hi = k + 2 * e + 1 < K ? t[c8 + 2 * e + 1][r] : 0u;
            w[e] = lo | (hi << 16);
        }
        *(u32x4*)(db + (int64_t)n * ld_dst + k) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// The same copy when K and N are multiples of 8 and the source rows are
// 16-byte aligned: each lane transposes one 8 x 8 block in registers (eight
// 16-byte loads along source rows, eight 16-byte stores along target rows),
// with no LDS round trip or barrier; a one-wave workgroup covers 64 x 64, so
// a small B still spreads over many CUs.
__global__ __launch_bounds__(64) void transpose8_bf16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                            int64_t s_src, uint16_t* __restrict__ dst,
                                                            int64_t ld_dst, int64_t s_dst, int K, int N) {
    const int lane = threadIdx.x;
    const int n = blockIdx.x * 64 + (lane & 7) * 8;
    const int k = blockIdx.y * 64 + (lane >> 3) * 8;
    if (n >= N || k >= K) return;   // K, N multiples of 8: whole blocks only
    const uint16_t* sb = src + (int64_t)blockIdx.z * s_src + (int64_t)k * ld_src + n;
    uint16_t* db = dst + (int64_t)blockIdx.z * s_dst + (int64_t)n * ld_dst + k;
    u32x4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = *(const u32x4*)(sb + (int64_t)r * ld_src);
    // target row c holds source column c: its dword e packs rows 2e and 2e+1
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = v[2 * e][c >> 1], hi = v[2 * e + 1][c >> 1];
            w[e] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        *(u32x4*)(db + (int64_t)c * ld_dst) = w;
    }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ C, int64_t ldc, int64_t sC, int M,
                                                        int N, int batch) {
    const int64_t per = (int64_t)M * N;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per * batch) return;
    const int b = (int)(idx / per);
    const int64_t e = idx % per;
    const int m = (int)(e / N), n = (int)(e % N);
    C[(int64_t)b * sC + (int64_t)m * ldc + n] = 0.0f;
}

// Sustained-rate probes for the offline stage.  mfma_probe: every wave keeps
// 16 independent 32x32x16 bf16 accumulations busy on random operands (MFMA
// power, hence clock, depends on operand bits).  copy_probe: a streaming
// 16-byte-per-lane copy.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x85EBCA6Bu;
    x ^= x >> 13;
    x *= 0xC2B2AE35u;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ uint32_t rand_bf16_pair(uint32_t x) {
    auto one = [](uint32_t h) { return ((h >> 31) << 15) | ((0x70u + (h >> 24) % 15u) << 7) | (h & 0x7fu); };
    return one(mix32(x)) | (one(mix32(x * 2654435761u + 1u)) << 16);
}

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters, uint32_t seed) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        u32x4 ua, ub;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t base = seed ^ (blockIdx.x * 4096u + threadIdx.x * 16u + s * 4u + e);
            ua[e] = rand_bf16_pair(base);
            ub[e] = rand_bf16_pair(base ^ 0x5bd1e995u);
        }
        a[s] = __builtin_bit_cast(bf16x8, ua);
        b[s] = __builtin_bit_cast(bf16x8, ub);
    }
    f32x16 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f32x16{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], b[(ks + j) & 3], acc[j], 0, 0, 0);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[j][r];
    out[blockIdx.x * 256 + threadIdx.x] = sum;
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = src[i];
}

// Read-only streaming probe: every lane reads 16-byte chunks, eight in
// flight, grid-stride over n chunks; one word per lane keeps the loads.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n, uint32_t* out) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < n; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; i += stride) {
        const u32x4 v = src[i];
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void fill_random_bf16_kernel(uint16_t* p, int64_t n, uint32_t seed) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        uint32_t x = (uint32_t)i * 0x9E3779B1u ^ seed;
        x ^= x >> 16;
        x *= 0x85EBCA6Bu;
        x ^= x >> 13;
        x *= 0xC2B2AE35u;
        x ^= x >> 16;
        // bf16 in [-1, 1): sign, exponent 0x70..0x7e, random mantissa
        const uint32_t sign = (x >> 31) << 15;
        const uint32_t expo = 0x70u + (x >> 24) % 15u;
        p[i] = (uint16_t)(sign | (expo << 7) | (x & 0x7fu));
    }
}

#endif  // helper kernels

// The library: tile shapes, wave layouts and LDS stage counts.  The large
// tiles run 8 waves (two per SIMD) so one wave's LDS waits overlap the
// other's MFMAs; 128x128 runs two 4-wave workgroups per CU.  With B as K x N
// the 256x256 tile uses 128 x 64 wave tiles: each wave then takes half as
// many B fragments through the slower transposed LDS reads as with 64 x 128.
using T_256x256 = Tile<256, 256, 64, 2, 4, 2>;
using T_256x128 = Tile<256, 128, 64, 4, 2, 2, true>;
using T_128x256 = Tile<128, 256, 64, 2, 4, 2>;
using T_128x128 = Tile<128, 128, 64, 2, 2, 2>;
using T_128x64 = Tile<128, 64, 64, 2, 2, 3>;
using T_64x128 = Tile<64, 128, 64, 2, 2, 3>;
using T_64x64 = Tile<64, 64, 64, 2, 2, 4>;
using T_32x128 = Tile<32, 128, 64, 1, 4, 4>;
using T_16x128 = Tile<16, 128, 64, 1, 4, 4>;
using T_16x256 = Tile<16, 256, 64, 1, 4, 4>;
using T_32x64 = Tile<32, 64, 64, 2, 2, 4>;
// 128 x 128 with four LDS stages: one workgroup per CU with three K steps of
// loads in flight instead of two workgroups with one each -- faster where K
// is deep or the tiles are few, slower on many shallow tiles.  Eight waves
// of 32 x 64 (4 x 2): twice the waves of a 2 x 2 layout issue the direct
// loads and the fragment reads of the one workgroup (8-15 % faster on the
// K x N shapes it serves, even to 8 % on N x K)
using T_128x128x4 = Tile<128, 128, 64, 4, 2, 4>;
// 256 x 256 on four waves of 128 x 128 accumulators (all 256 AGPRs), one
// wave per SIMD: each fragment read from LDS feeds four MFMAs instead of
// two, halving the LDS bytes per MFMA of the eight-wave form.
using T_256x256w4 = Tile<256, 256, 64, 2, 2, 2>;
// the 64 x 64, 64 x 128 and 128 x 64 tiles with two LDS stages: half the
// LDS of the three- and four-stage forms, so more workgroups share a CU --
// faster on most shapes, slower where deep K on few tiles needs the deeper
// pipeline
using T_64x64x2 = Tile<64, 64, 64, 2, 2, 2>;
using T_64x128x2 = Tile<64, 128, 64, 2, 2, 2>;
using T_128x64x2 = Tile<128, 64, 64, 2, 2, 2>;
// skinny-M tiles with the K range split across 4 waves (uK = 256 per
// workgroup step; see WSplit)
using W_16x64 = WSplit<16, 64, 4, 3, false>;
using W_32x64 = WSplit<32, 64, 4, 3, false>;
using W_64x64 = WSplit<64, 64, 4, 2, false>;
using W_16x128 = WSplit<16, 128, 4, 2, false>;
using X_16x64 = WSplit<16, 64, 4, 3, true>;
using X_32x64 = WSplit<32, 64, 4, 3, true>;
using X_64x64 = WSplit<64, 64, 4, 2, true>;
using X_16x128 = WSplit<16, 128, 4, 2, true>;
// the same tiles for B given as N x K
using U_256x256 = Tile<256, 256, 64, 4, 2, 2, false, true>;
using U_256x128 = Tile<256, 128, 64, 4, 2, 2, true, true>;
using U_128x256 = Tile<128, 256, 64, 2, 4, 2, false, true>;
using U_128x128 = Tile<128, 128, 64, 2, 2, 2, false, true>;
using U_128x64 = Tile<128, 64, 64, 2, 2, 3, false, true>;
using U_64x128 = Tile<64, 128, 64, 2, 2, 3, false, true>;
using U_64x64 = Tile<64, 64, 64, 2, 2, 4, false, true>;
// the single-kernel 64 x 128 tile runs eight waves of 32 x 32 (2 x 4): 4-26 %
// faster than four waves of 32 x 64 on the shapes it serves, most on few
// tiles and on one-step (K = 64) batches; the two-tile kernels keep the
// four-wave form, the workgroup size of their 128 x 128 partner (the 64 x 64
// tile lost 20-28 % with eight waves and keeps four)
using T_64x128w8 = Tile<64, 128, 64, 2, 4, 3>;
using U_64x128w8 = Tile<64, 128, 64, 2, 4, 3, false, true>;
// likewise the single-kernel 128 x 64 tile (eight waves of 32 x 32, 4 x 2:
// 4-10 % faster), and the K x N two-stage 64 x 128 and 128 x 64 tiles (even
// to 5 % faster on GEMMs, 14-17 % on one-step K = 64 batches; their N x K
// forms gained nothing and keep four waves, as does the two-stage 64 x 64
// tile, 6-43 % slower with eight)
using T_128x64w8 = Tile<128, 64, 64, 4, 2, 3>;
using U_128x64w8 = Tile<128, 64, 64, 4, 2, 3, false, true>;
using T_64x128x2w8 = Tile<64, 128, 64, 2, 4, 2>;
using T_128x64x2w8 = Tile<128, 64, 64, 4, 2, 2>;
using U_32x128 = Tile<32, 128, 64, 1, 4, 4, false, true>;
using U_16x128 = Tile<16, 128, 64, 1, 4, 4, false, true>;
using U_16x256 = Tile<16, 256, 64, 1, 4, 4, false, true>;
using U_32x64 = Tile<32, 64, 64, 2, 2, 4, false, true>;
using U_128x128x4 = Tile<128, 128, 64, 4, 2, 4, false, true>;
using U_256x256w4 = Tile<256, 256, 64, 2, 2, 2, false, true>;
using U_64x64x2 = Tile<64, 64, 64, 2, 2, 2, false, true>;
using U_64x128x2 = Tile<64, 128, 64, 2, 2, 2, false, true>;
using U_128x64x2 = Tile<128, 64, 64, 2, 2, 2, false, true>;

#if MKP_PART == 0 || MKP_PART == 1
#define MKP_KERNEL(NAME, T)                                                                               \
    {                                                                                                      \
        NAME, T::BM, T::BN, T::BK, T::NT, T::LDS, T::FUSED, T::BT, (const void*)&gemm_tile_kernel<T>, \
            &launch_tile<T>                                                                                \
    }
#define MKP_WSPLIT(NAME, W) \
    { NAME, W::BM, W::BN, W::BK, W::NT, W::LDS, false, W::BT, (const void*)&gemm_wsplit_kernel<W>, &launch_wsplit<W> }

const KernelInfo g_kernels[] = {
    MKP_KERNEL("m256n256k64", T_256x256),
    MKP_KERNEL("m256n128k64", T_256x128),
    MKP_KERNEL("m128n256k64", T_128x256),
    MKP_KERNEL("m128n128k64", T_128x128),
    MKP_KERNEL("m128n64k64", T_128x64w8),
    MKP_KERNEL("m64n128k64", T_64x128w8),
    MKP_KERNEL("m64n64k64", T_64x64),
    MKP_KERNEL("m32n128k64", T_32x128),
    MKP_KERNEL("m16n128k64", T_16x128),
    MKP_KERNEL("m16n256k64", T_16x256),
    MKP_KERNEL("m32n64k64", T_32x64),
    MKP_KERNEL("m128n128k64x4", T_128x128x4),
    MKP_KERNEL("m256n256k64w4", T_256x256w4),
    MKP_KERNEL("m64n64k64x2", T_64x64x2),
    MKP_KERNEL("m64n128k64x2", T_64x128x2w8),
    MKP_KERNEL("m128n64k64x2", T_128x64x2w8),
    MKP_WSPLIT("m16n64k256", W_16x64),
    MKP_WSPLIT("m32n64k256", W_32x64),
    MKP_WSPLIT("m64n64k256", W_64x64),
    MKP_WSPLIT("m16n128k256", W_16x128),
    MKP_KERNEL("m256n256k64_nk", U_256x256),
    MKP_KERNEL("m256n128k64_nk", U_256x128),
    MKP_KERNEL("m128n256k64_nk", U_128x256),
    MKP_KERNEL("m128n128k64_nk", U_128x128),
    MKP_KERNEL("m128n64k64_nk", U_128x64w8),
    MKP_KERNEL("m64n128k64_nk", U_64x128w8),
    MKP_KERNEL("m64n64k64_nk", U_64x64),
    MKP_KERNEL("m32n128k64_nk", U_32x128),
    MKP_KERNEL("m16n128k64_nk", U_16x128),
    MKP_KERNEL("m16n256k64_nk", U_16x256),
    MKP_KERNEL("m32n64k64_nk", U_32x64),
    MKP_KERNEL("m128n128k64x4_nk", U_128x128x4),
    MKP_KERNEL("m256n256k64w4_nk", U_256x256w4),
    MKP_KERNEL("m64n64k64x2_nk", U_64x64x2),
    MKP_KERNEL("m64n128k64x2_nk", U_64x128x2),
    MKP_KERNEL("m128n64k64x2_nk", U_128x64x2),
    MKP_WSPLIT("m16n64k256_nk", X_16x64),
    MKP_WSPLIT("m32n64k256_nk", X_32x64),
    MKP_WSPLIT("m64n64k256_nk", X_64x64),
    MKP_WSPLIT("m16n128k256_nk", X_16x128),
};

#endif  // single-tile registry

// The convolution forms of the N x K tiles (implicit GEMM; same tiles).
using V_256x256 = Tile<256, 256, 64, 4, 2, 2, false, true, true>;
using V_256x128 = Tile<256, 128, 64, 4, 2, 2, true, true, true>;
using V_128x256 = Tile<128, 256, 64, 2, 4, 2, false, true, true>;
using V_128x128 = Tile<128, 128, 64, 2, 2, 2, false, true, true>;
using V_128x64 = Tile<128, 64, 64, 2, 2, 3, false, true, true>;
using V_64x128 = Tile<64, 128, 64, 2, 2, 3, false, true, true>;
using V_64x64 = Tile<64, 64, 64, 2, 2, 4, false, true, true>;
using V_32x128 = Tile<32, 128, 64, 1, 4, 4, false, true, true>;
using V_16x128 = Tile<16, 128, 64, 1, 4, 4, false, true, true>;
using V_16x256 = Tile<16, 256, 64, 1, 4, 4, false, true, true>;
using V_32x64 = Tile<32, 64, 64, 2, 2, 4, false, true, true>;
// (the convolution form keeps four waves of 64 x 64: with eight, every wave
// repeats the filter-tap bookkeeping of the gather, and the 3 x 3 layers ran
// 8-14 % slower)
using V_128x128x4 = Tile<128, 128, 64, 2, 2, 4, false, true, true>;
using V_256x256w4 = Tile<256, 256, 64, 2, 2, 2, false, true, true>;
using V_64x64x2 = Tile<64, 64, 64, 2, 2, 2, false, true, true>;
using V_64x128x2 = Tile<64, 128, 64, 2, 2, 2, false, true, true>;
using V_128x64x2 = Tile<128, 64, 64, 2, 2, 2, false, true, true>;

#if MKP_PART == 0 || MKP_PART == 4
#define MKP_CONV(TWIN, T) \
    { TWIN, (const void*)&gemm_tile_kernel<T>, &launch_tile<T> }
const ConvInfo g_conv[] = {
    MKP_CONV("m256n256k64_nk", V_256x256), MKP_CONV("m256n128k64_nk", V_256x128),
    MKP_CONV("m128n256k64_nk", V_128x256), MKP_CONV("m128n128k64_nk", V_128x128),
    MKP_CONV("m128n64k64_nk", V_128x64),   MKP_CONV("m64n128k64_nk", V_64x128),
    MKP_CONV("m64n64k64_nk", V_64x64),     MKP_CONV("m32n128k64_nk", V_32x128),
    MKP_CONV("m16n128k64_nk", V_16x128),   MKP_CONV("m16n256k64_nk", V_16x256),
    MKP_CONV("m32n64k64_nk", V_32x64),     MKP_CONV("m128n128k64x4_nk", V_128x128x4),
    MKP_CONV("m256n256k64w4_nk", V_256x256w4), MKP_CONV("m64n64k64x2_nk", V_64x64x2),
    MKP_CONV("m64n128k64x2_nk", V_64x128x2),   MKP_CONV("m128n64k64x2_nk", V_128x64x2),
};
#endif

// Pairs of tiles that can share a launch (same workgroup size and resident
// workgroups per CU): a large tile for the region of whole waves and a
// smaller one for the rest, in both B layouts.
#define MKP_DUAL(N1, T1, N2, T2) \
    { N1, N2, (const void*)&gemm_dual_kernel<T1, T2>, &launch_dual<T1, T2> }

#if MKP_PART == 0 || MKP_PART == 2
const DualInfo g_duals_kn[] = {
    MKP_DUAL("m128n128k64", T_128x128, "m64n64k64", T_64x64),
    MKP_DUAL("m128n128k64", T_128x128, "m64n128k64", T_64x128),
    MKP_DUAL("m128n128k64", T_128x128, "m128n64k64", T_128x64),
    MKP_DUAL("m128n128k64", T_128x128, "m16n128k64", T_16x128),
    MKP_DUAL("m128n64k64", T_128x64, "m64n64k64", T_64x64),
    MKP_DUAL("m64n128k64", T_64x128, "m64n64k64", T_64x64),
    MKP_DUAL("m256n256k64", T_256x256, "m256n128k64", T_256x128),
    MKP_DUAL("m256n256k64", T_256x256, "m128n256k64", T_128x256),
};
#endif
#if MKP_PART == 0 || MKP_PART == 3
const DualInfo g_duals_nk[] = {
    MKP_DUAL("m128n128k64_nk", U_128x128, "m64n64k64_nk", U_64x64),
    MKP_DUAL("m128n128k64_nk", U_128x128, "m64n128k64_nk", U_64x128),
    MKP_DUAL("m128n128k64_nk", U_128x128, "m128n64k64_nk", U_128x64),
    MKP_DUAL("m128n128k64_nk", U_128x128, "m16n128k64_nk", U_16x128),
    MKP_DUAL("m128n64k64_nk", U_128x64, "m64n64k64_nk", U_64x64),
    MKP_DUAL("m64n128k64_nk", U_64x128, "m64n64k64_nk", U_64x64),
    MKP_DUAL("m256n256k64_nk", U_256x256, "m256n128k64_nk", U_256x128),
    MKP_DUAL("m256n256k64_nk", U_256x256, "m128n256k64_nk", U_128x256),
};
#endif

}  // namespace

#if MKP_PART == 0 || MKP_PART == 4
int conv_count() { return (int)(sizeof(g_conv) / sizeof(g_conv[0])); }
const ConvInfo& conv_info(int i) { return g_conv[i]; }
#endif

// the pair tables of the two-tile translation units
const DualInfo* duals_kn(int* n);
const DualInfo* duals_nk(int* n);
#if MKP_PART == 0 || MKP_PART == 2
const DualInfo* duals_kn(int* n) {
    *n = (int)(sizeof(g_duals_kn) / sizeof(g_duals_kn[0]));
    return g_duals_kn;
}
#endif
#if MKP_PART == 0 || MKP_PART == 3
const DualInfo* duals_nk(int* n) {
    *n = (int)(sizeof(g_duals_nk) / sizeof(g_duals_nk[0]));
    return g_duals_nk;
}
#endif
#if MKP_PART == 0 || MKP_PART == 1
int dual_count() {
    int a = 0, b = 0;
    duals_kn(&a);
    duals_nk(&b);
    return a + b;
}
const DualInfo& dual_info(int i) {
    int a = 0, b = 0;
    const DualInfo* kn = duals_kn(&a);
    const DualInfo* nk = duals_nk(&b);
    return i < a ? kn[i] : nk[i - a];
}
#endif

#if MKP_PART == 0 || MKP_PART == 1
// Device memory of the allocation-free entry point: a fixed array in the
// code object (zero at load, held by every GPU the library runs on until the
// process ends), serving as that call's split-K partials and staging copies.
// Host code never passes the name itself (on the host it only stands for
// the symbol): static_scratch() gives each device's own address, looked up
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(int dev, void** out) {
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    std::lock_guard<std::mutex> lk(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
    ptrs.emplace(dev, p);
    *out = p;
    return hipSuccess;
}

LaunchEvents& launch_events() {
    thread_local LaunchEvents slot;
    return slot;
}

int kernel_count() { return (int)(sizeof(g_kernels) / sizeof(g_kernels[0])); }
const KernelInfo& kernel_info(int i) { return g_kernels[i]; }
int kernel_find(const char* name) {
    for (int i = 0; i < kernel_count(); ++i)
        if (__builtin_strcmp(g_kernels[i].name, name) == 0) return i;
    return -1;
}

hipError_t launch_splitk_reduce(const float* W, int splits, int64_t sWsplit, int64_t sWbatch, int64_t ldw, float* C,
                                int64_t ldc, int64_t sC, int M, int N, int batch, int vec, hipStream_t st,
                                const KEpi* epi) {
    const int64_t items = (int64_t)M * ((N + 3) / 4) * batch;
    if (items == 0) return hipSuccess;
    if (items > (int64_t)UINT32_MAX * 256) return hipErrorInvalidValue;
    dim3 grid((unsigned)((items + 255) / 256));
    if (epi)
        return launch_kernel(splitk_reduce_kernel<true>, grid, dim3(256), st, W, splits, sWsplit, sWbatch, ldw, C, ldc,
                             sC, M, N, batch, vec, *epi);
    return launch_kernel(splitk_reduce_kernel<false>, grid, dim3(256), st, W, splits, sWsplit, sWbatch, ldw, C, ldc, sC,
                         M, N, batch, vec, KEpi{});
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t ld_src, int64_t s_src, uint16_t* dst, int64_t ld_dst,
                                 int64_t s_dst, int K, int N, int batch, bool src_vec, hipStream_t st) {
    if (batch > 65535 || (ld_dst + 63) / 64 > 65535 || ld_dst % 8 != 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((ld_dst + 63) / 64), (unsigned)batch);
    if (src_vec && K % 8 == 0 && N % 8 == 0 && ld_dst == K)
        return launch_kernel(transpose8_bf16_kernel, grid, dim3(64), st, src, ld_src, s_src, dst, ld_dst, s_dst, K, N);
    if (src_vec)
        return launch_kernel(transpose_bf16_kernel<true>, grid, dim3(256), st, src, ld_src, s_src, dst, ld_dst, s_dst, K,
                             N);
    return launch_kernel(transpose_bf16_kernel<false>, grid, dim3(256), st, src, ld_src, s_src, dst, ld_dst, s_dst, K,
                         N);
}

hipError_t launch_zero_fill(float* C, int64_t ldc, int64_t sC, int M, int N, int batch, hipStream_t st) {
    const int64_t items = (int64_t)M * N * batch;
    dim3 grid((unsigned)((items + 255) / 256));
    return launch_kernel(zero_fill_kernel, grid, dim3(256), st, C, ldc, sC, M, N, batch);
}

hipError_t launch_pack_rows(const uint16_t* src, int64_t ld_src, int64_t stride_src, uint16_t* dst, int64_t ld_dst,
                            int rows, int cols, int batch, hipStream_t st) {
    const int64_t items = (int64_t)rows * (ld_dst >> 3) * batch;
    return launch_kernel(pack_rows_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), st, src, ld_src,
                         stride_src, dst, ld_dst, rows, cols, batch);
}

hipError_t launch_mfma_probe(float* out, int blocks, int iters, hipStream_t st) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, st, out, iters, 0x9e3779b9u);
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, int blocks, hipStream_t st) {
    hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4*)src, (u32x4*)dst, bytes / 16);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, st, (const u32x4*)src, bytes / 16, out);
    return hipGetLastError();
}

hipError_t launch_fill_random_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t st) {
    hipLaunchKernelGGL(fill_random_bf16_kernel, dim3(1024), dim3(256), 0, st, p, n, seed);
    return hipGetLastError();
}

#endif  // part 1

}  // namespace mkp
