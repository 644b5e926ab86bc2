// CDNA4 (gfx950) micro-kernel library.
//
// Every micro-kernel is one fixed uM x uN x uK tile; a workgroup runs one
// pipeline task: it walks its K range in uK steps, each step loading the A
// (uM x uK) and B (uK x uN) tiles from HBM into LDS, then running bf16 MFMAs
// on them with fp32 accumulation, and finally writes the fp32 tile back
// (MikPoly page, section 3 "micro-kernel performance model": load to local
// memory, compute with intermediates kept local, write back).  Start
// addresses, extents and K trip counts are run-time arguments (section 4).
// Edge tiles are predicated element by element, so any shape is covered
// without padding the operands ("partial padding", section 3, polymerization
// strategy).
//
// Data path per K step (register-staged double buffering, one barrier):
//   * A rows are K-contiguous, which is what the MFMA operand wants: 128-bit
//     global loads go straight into a K-major LDS tile.
//   * B rows are N-contiguous; each thread loads a 4(k) x 8(n) block with
//     four 128-bit loads, transposes it in registers and stores it into an
//     N-major (K-contiguous) LDS tile, so both MFMA operands are read with
//     one 128-bit LDS read per lane.
//   * LDS rows are 16-byte-chunk XOR swizzled so the 16 lanes that read one
//     MFMA fragment hit distinct banks.
//   * v_mfma_f32_16x16x32_bf16 is issued with the B^T fragment as the first
//     operand and the A^T fragment as the second, so each lane's four
//     results are four consecutive columns of one C row: one 128-bit store.
#include "kernels.h"

#include <hip/hip_runtime.h>

namespace mkp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int BK>
__device__ __forceinline__ int swz(int row);
// 128-byte rows (8 chunks): rows r and r+8 differ in chunk parity, rows r
// and r+1 fall in different halves of a 256-byte bank window.
template <>
__device__ __forceinline__ int swz<64>(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// 256-byte rows (16 chunks)
template <>
__device__ __forceinline__ int swz<128>(int row) { return row & 15; }

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int ROWB = BK * 2;             // bytes per LDS row
    static constexpr int CPR = BK / 8;              // 16-byte chunks per row
    static constexpr int A_CH = BM * CPR;           // A chunks per tile
    static constexpr int B_Q = (BK / 4) * (BN / 8); // B 4x8 blocks per tile
    static constexpr int NA = (A_CH + NT - 1) / NT;
    static constexpr int NB = (B_Q + NT - 1) / NT;
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BN * ROWB;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = 2 * STAGE;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BK == 64 || BK == 128, "uK must be 64 or 128");
    static_assert(LDS <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// Up to 8 consecutive bf16 values, element-wise (any alignment); missing
// elements read as zero.  Nothing is read when nvalid <= 0.
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

__device__ __forceinline__ uint32_t half16(uint32_t x, int hi) { return hi ? (x >> 16) : (x & 0xffffu); }

template <class T>
struct Pipe {
    u32x4 ra[T::NA];
    u32x4 rb[T::NB][4];

    // Global -> registers for the K step starting at k0.
    // fast: the whole tile and step are in range and rows are 16-byte aligned.
    __device__ __forceinline__ void load(const uint16_t* __restrict__ A, int64_t lda,
                                         const uint16_t* __restrict__ B, int64_t ldb, int k0, int kend,
                                         int Mr, int Nr, bool fast, bool vecA, bool vecB, int tid) {
#pragma unroll
        for (int i = 0; i < T::NA; ++i) {
            const int q = tid + i * T::NT;
            if (T::A_CH % T::NT == 0 || q < T::A_CH) {
                const int row = q / T::CPR, kc = q % T::CPR;
                const int k = k0 + kc * 8;
                const uint16_t* p = A + (int64_t)row * lda + k;
                if (fast) {
                    ra[i] = *(const u32x4*)p;
                } else if (row < Mr && k < kend) {
                    ra[i] = (vecA && k + 8 <= kend) ? *(const u32x4*)p : load8_elems(p, kend - k);
                } else {
                    ra[i] = zero4();
                }
            }
        }
#pragma unroll
        for (int i = 0; i < T::NB; ++i) {
            const int q = tid + i * T::NT;
            if (T::B_Q % T::NT == 0 || q < T::B_Q) {
                const int kq = q % (T::BK / 4), nq = q / (T::BK / 4);
                const int n = nq * 8;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int k = k0 + kq * 4 + j;
                    const uint16_t* p = B + (int64_t)k * ldb + n;
                    if (fast) {
                        rb[i][j] = *(const u32x4*)p;
                    } else if (k < kend && n < Nr) {
                        rb[i][j] = (vecB && n + 8 <= Nr) ? *(const u32x4*)p : load8_elems(p, Nr - n);
                    } else {
                        rb[i][j] = zero4();
                    }
                }
            }
        }
    }

    // Registers -> LDS stage (A K-major as loaded, B transposed to N-major).
    __device__ __forceinline__ void store(unsigned char* st, int tid) {
#pragma unroll
        for (int i = 0; i < T::NA; ++i) {
            const int q = tid + i * T::NT;
            if (T::A_CH % T::NT == 0 || q < T::A_CH) {
                const int row = q / T::CPR, kc = q % T::CPR;
                *(u32x4*)(st + row * T::ROWB + ((kc ^ swz<T::BK>(row)) << 4)) = ra[i];
            }
        }
        unsigned char* sb = st + T::A_BYTES;
#pragma unroll
        for (int i = 0; i < T::NB; ++i) {
            const int q = tid + i * T::NT;
            if (T::B_Q % T::NT == 0 || q < T::B_Q) {
                const int kq = q % (T::BK / 4), nq = q / (T::BK / 4);
                const int c = kq >> 1, h = kq & 1;
#pragma unroll
                for (int nn = 0; nn < 8; ++nn) {
                    const int n = nq * 8 + nn;
                    const int w = nn >> 1, hi = nn & 1;
                    const uint32_t d0 = half16(rb[i][0][w], hi) | (half16(rb[i][1][w], hi) << 16);
                    const uint32_t d1 = half16(rb[i][2][w], hi) | (half16(rb[i][3][w], hi) << 16);
                    *(u32x2*)(sb + n * T::ROWB + ((c ^ swz<T::BK>(n)) << 4) + h * 8) = u32x2{d0, d1};
                }
            }
        }
    }
};

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

template <class T>
__global__ __launch_bounds__(T::NT) void gemm_tile_kernel(KArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % T::WGM, wn = wave / T::WGM;

    int tm, tn, split, b;
    map_tile<8>(blockIdx.x, gridDim.x, args.tiles_m, args.tiles_n, args.splits, tm, tn, split, b);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const uint16_t* __restrict__ A = args.A + (int64_t)b * args.sA + (int64_t)m0 * args.lda;
    const uint16_t* __restrict__ B = args.B + (int64_t)b * args.sB + n0;
    const int Mr = args.M - m0, Nr = args.N - n0;
    const int kbeg = split * args.steps_per_split * T::BK;
    const int kend = min(args.K, kbeg + args.steps_per_split * T::BK);
    const int nsteps = (kend - kbeg + T::BK - 1) / T::BK;

    const bool vecA = args.flags & KF_VEC_A, vecB = args.flags & KF_VEC_B;
    const bool tile_fast = vecA && vecB && Mr >= T::BM && Nr >= T::BN;

    f32x4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Pipe<T> pipe;
    {
        const bool fast = tile_fast && kbeg + T::BK <= kend;
        pipe.load(A, args.lda, B, args.ldb, kbeg, kend, Mr, Nr, fast, vecA, vecB, tid);
        pipe.store(smem, tid);
    }
    __syncthreads();

    const int frow = lane & 15, fchunk = lane >> 4;
    for (int s = 0; s < nsteps; ++s) {
        unsigned char* cur = smem + (s & 1) * T::STAGE;
        const bool more = s + 1 < nsteps;
        if (more) {
            const int k0 = kbeg + (s + 1) * T::BK;
            const bool fast = tile_fast && k0 + T::BK <= kend;
            pipe.load(A, args.lda, B, args.ldb, k0, kend, Mr, Nr, fast, vecA, vecB, tid);
        }
#pragma unroll
        for (int ks = 0; ks < T::BK / 32; ++ks) {
            const int c = ks * 4 + fchunk;
            u32x4 xb[T::FN], ya[T::FM];
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const int row = wn * T::WTN + j * 16 + frow;
                xb[j] = *(const u32x4*)(cur + T::A_BYTES + row * T::ROWB + ((c ^ swz<T::BK>(row)) << 4));
            }
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const int row = wm * T::WTM + i * 16 + frow;
                ya[i] = *(const u32x4*)(cur + row * T::ROWB + ((c ^ swz<T::BK>(row)) << 4));
            }
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, xb[j]), __builtin_bit_cast(bf16x8, ya[i]), acc[i][j], 0, 0, 0);
        }
        if (more) pipe.store(smem + ((s + 1) & 1) * T::STAGE, tid);
        __syncthreads();
    }

    // Epilogue: lane holds C[m][n..n+3] of each fragment.
    float* __restrict__ C = args.C + (int64_t)b * args.sC + (int64_t)split * args.sCsplit +
                            (int64_t)m0 * args.ldc + n0;
    const bool vecC = args.flags & KF_VEC_C;
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
        const int m = wm * T::WTM + i * 16 + frow;
        if (m >= Mr) continue;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int n = wn * T::WTN + j * 16 + fchunk * 4;
            float* p = C + (int64_t)m * args.ldc + n;
            if (vecC && n + 4 <= Nr) {
                *(f32x4*)p = acc[i][j];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < Nr) p[r] = acc[i][j][r];
            }
        }
    }
}

template <class T>
hipError_t launch_tile(const KArgs& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL(gemm_tile_kernel<T>, grid, dim3(T::NT), 0, st, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ W, int splits, int64_t sWs,
                                                            int64_t sWb, int64_t ldw, float* __restrict__ C,
                                                            int64_t ldc, int64_t sC, int M, int N, int batch,
                                                            int vec) {
    const int nq = (N + 3) >> 2;
    const int64_t per = (int64_t)M * nq;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= per * batch) return;
    const int b = (int)(idx / per);
    const int64_t e = idx % per;
    const int m = (int)(e / nq);
    const int n = (int)(e % nq) * 4;
    const float* w = W + (int64_t)b * sWb + (int64_t)m * ldw + n;
    f32x4 s = *(const f32x4*)w;
    for (int z = 1; z < splits; ++z) s += *(const f32x4*)(w + (int64_t)z * sWs);
    float* p = C + (int64_t)b * sC + (int64_t)m * ldc + n;
    if (vec && n + 4 <= N) {
        *(f32x4*)p = s;
    } else {
        for (int r = 0; r < 4; ++r)
            if (n + r < N) p[r] = s[r];
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

// The library: tile shapes and their wave layouts.
using T_256x256 = Tile<256, 256, 64, 2, 2>;
using T_256x128 = Tile<256, 128, 64, 2, 2>;
using T_128x256 = Tile<128, 256, 64, 2, 2>;
using T_128x128 = Tile<128, 128, 64, 2, 2>;
using T_128x64 = Tile<128, 64, 64, 2, 2>;
using T_64x128 = Tile<64, 128, 64, 2, 2>;
using T_64x64 = Tile<64, 64, 64, 2, 2>;
using T_32x128 = Tile<32, 128, 128, 1, 4>;
using T_16x128 = Tile<16, 128, 128, 1, 4>;
using T_16x256 = Tile<16, 256, 128, 1, 4>;
using T_32x64 = Tile<32, 64, 128, 2, 2>;

#define MKP_KERNEL(NAME, T) \
    { NAME, T::BM, T::BN, T::BK, T::NT, T::LDS, (const void*)&gemm_tile_kernel<T>, &launch_tile<T> }

const KernelInfo g_kernels[] = {
    MKP_KERNEL("m256n256k64", T_256x256),
    MKP_KERNEL("m256n128k64", T_256x128),
    MKP_KERNEL("m128n256k64", T_128x256),
    MKP_KERNEL("m128n128k64", T_128x128),
    MKP_KERNEL("m128n64k64", T_128x64),
    MKP_KERNEL("m64n128k64", T_64x128),
    MKP_KERNEL("m64n64k64", T_64x64),
    MKP_KERNEL("m32n128k128", T_32x128),
    MKP_KERNEL("m16n128k128", T_16x128),
    MKP_KERNEL("m16n256k128", T_16x256),
    MKP_KERNEL("m32n64k128", T_32x64),
};

}  // namespace

int kernel_count() { return (int)(sizeof(g_kernels) / sizeof(g_kernels[0])); }
const KernelInfo& kernel_info(int i) { return g_kernels[i]; }
int kernel_find(const char* name) {
    for (int i = 0; i < kernel_count(); ++i)
        if (__builtin_strcmp(g_kernels[i].name, name) == 0) return i;
    return -1;
}

hipError_t launch_splitk_reduce(const float* W, int splits, int64_t sWsplit, int64_t sWbatch, int64_t ldw, float* C,
                                int64_t ldc, int64_t sC, int M, int N, int batch, int vec, hipStream_t st) {
    const int64_t items = (int64_t)M * ((N + 3) / 4) * batch;
    dim3 grid((unsigned)((items + 255) / 256));
    hipLaunchKernelGGL(splitk_reduce_kernel, grid, dim3(256), 0, st, W, splits, sWsplit, sWbatch, ldw, C, ldc, sC, M,
                       N, batch, vec);
    return hipGetLastError();
}

hipError_t launch_zero_fill(float* C, int64_t ldc, int64_t sC, int M, int N, int batch, hipStream_t st) {
    const int64_t items = (int64_t)M * N * batch;
    dim3 grid((unsigned)((items + 255) / 256));
    hipLaunchKernelGGL(zero_fill_kernel, grid, dim3(256), 0, st, C, ldc, sC, M, N, batch);
    return hipGetLastError();
}

hipError_t launch_fill_random_bf16(uint16_t* p, int64_t n, uint32_t seed, hipStream_t st) {
    hipLaunchKernelGGL(fill_random_bf16_kernel, dim3(1024), dim3(256), 0, st, p, n, seed);
    return hipGetLastError();
}

}  // namespace mkp
