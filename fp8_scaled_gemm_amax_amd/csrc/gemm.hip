// gemm.hip - scaled FP8 GEMM on gfx950 matrix cores, dense and grouped (MoE).
//
//   d[i, j] = out( fp32acc( sum_k a[i, k] * b[j, k] ) * sa_i * sb_j )
//
// Sources: "FP8 Training on AMD GPUs with TorchTitan and TorchAO" (rowwise FP8
// linear layers, FP8 grouped GEMM for MoE); "FP8 training for Flux models",
// section "Configuration" (e4m3, and "hybrid" = e4m3 activations/weights with
// e5m2 gradients; FP8 wgrad).
//
// Both operands are K-contiguous (a: [m x k], b: [n x k]). A workgroup of four
// 64-lane wavefronts computes a BM x BN tile; each wavefront owns a 64 x 64
// quarter as 2 x 2 blocks of v_mfma_f32_32x32x64_f8f6f4 (fp32 accumulators).
// K advances in steps of 128 bytes through LDS; the next step's global loads
// are issued before the current step's matrix instructions (register
// prefetch). LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
// the row, so that the fragment reads of 32 consecutive rows spread over banks.
#include "fp8_device.hpp"
#include "kernels.hpp"

namespace fp8amax {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 16;                            // 8
constexpr int kLoadsA = BM * kChunksPerRow / kThreads;            // 4
constexpr int kLoadsB = BN * kChunksPerRow / kThreads;            // 4

// Matrix-core operand format selectors: 0 = e4m3 (fp8), 1 = e5m2 (bf8).
template <int F> struct MfmaFmt;
template <> struct MfmaFmt<kE4M3> { static constexpr int v = 0; };
template <> struct MfmaFmt<kE5M2> { static constexpr int v = 1; };

struct TileArgs {
    const uint8_t* a;   // first row of the tile's row range
    const uint8_t* b;
    int64_t lda, ldb;
    int64_t m_rows;     // valid rows of a from `a` on (tile-relative upper bound)
    int64_t n_rows;     // valid rows of b
    int64_t k;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ (row & 7)); }

template <int LOADS>
__device__ __forceinline__ void load_tile(uint4 (&r)[LOADS], const uint8_t* base, int64_t ld, int64_t valid_rows,
                                          int64_t k0, int64_t k) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int c = threadIdx.x + i * kThreads;
        const int row = c >> 3, kc = c & 7;
        const int64_t kk = k0 + kc * 16;
        if (row < valid_rows && kk < k)
            r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + kk);
        else
            r[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

template <int LOADS>
__device__ __forceinline__ void store_tile(const uint4 (&r)[LOADS], uint4* lds) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int c = threadIdx.x + i * kThreads;
        lds[swz(c >> 3, c & 7)] = r[i];
    }
}

// Fragment of the 32x32x64 instruction: lane l supplies row (l % 32) of its
// 32-row block and 32 consecutive K bytes starting at (l / 32) * 32 of the
// 64-wide K slice kk. The same map is used for a and b, so the contraction
// pairs equal K indices whatever order the instruction sums them in.
__device__ __forceinline__ v8i load_frag(const uint4* lds, int row, int kk) {
    const int lane = threadIdx.x & 63;
    const int c0 = kk * 4 + (lane >> 5) * 2;
    const uint4 lo = lds[swz(row, c0)];
    const uint4 hi = lds[swz(row, c0 + 1)];
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

// One BM x BN output tile: acc[mi][ni] holds the wavefront's 32x32 block (mi, ni).
template <int FA, int FB>
__device__ __forceinline__ void mma_tile(const TileArgs& t, v16f (&acc)[2][2], uint4* As, uint4* Bs) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    const int64_t nk = (t.k + BK - 1) / BK;
    uint4 ra[kLoadsA], rb[kLoadsB];
    if (nk > 0) {
        load_tile<kLoadsA>(ra, t.a, t.lda, t.m_rows, 0, t.k);
        load_tile<kLoadsB>(rb, t.b, t.ldb, t.n_rows, 0, t.k);
    }
    for (int64_t kt = 0; kt < nk; ++kt) {
        __syncthreads();
        store_tile<kLoadsA>(ra, As);
        store_tile<kLoadsB>(rb, Bs);
        __syncthreads();
        if (kt + 1 < nk) {
            load_tile<kLoadsA>(ra, t.a, t.lda, t.m_rows, (kt + 1) * BK, t.k);
            load_tile<kLoadsB>(rb, t.b, t.ldb, t.n_rows, (kt + 1) * BK, t.k);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi) fa[mi] = load_frag(As, wm * 64 + mi * 32 + (lane & 31), kk);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni) fb[ni] = load_frag(Bs, wn * 64 + ni * 32 + (lane & 31), kk);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[mi], fb[ni], acc[mi][ni], MfmaFmt<FA>::v, MfmaFmt<FB>::v, 0, 0, 0, 0);
        }
    }
}

// Epilogue: accumulator register r of block (mi, ni) in lane l holds row
// 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
template <bool OUT_F32>
__device__ __forceinline__ void store_tile_out(const v16f (&acc)[2][2], void* d, int64_t ldd, int64_t row0,
                                               int64_t rows_valid, int64_t col0, int64_t cols_valid,
                                               const float* sa, int sa_vec, const float* sb, int sb_vec) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int lc = wn * 64 + ni * 32 + (lane & 31);
        if (lc >= cols_valid) continue;
        const float sbj = sb[sb_vec ? col0 + lc : 0];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (lr >= rows_valid) continue;
                const float sai = sa[sa_vec ? row0 + lr : 0];
                const float v = acc[mi][ni][r] * sai * sbj;
                const int64_t off = (row0 + lr) * ldd + col0 + lc;
                if (OUT_F32)
                    reinterpret_cast<float*>(d)[off] = v;
                else
                    reinterpret_cast<uint16_t*>(d)[off] = (uint16_t)f32_to_bf16(v);
            }
        }
    }
}

template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_gemm(const uint8_t* __restrict__ a, int64_t lda,
                                                   const uint8_t* __restrict__ b, int64_t ldb, int64_t m, int64_t n,
                                                   int64_t k, const float* __restrict__ sa, int sa_vec,
                                                   const float* __restrict__ sb, int sb_vec, void* __restrict__ d,
                                                   int64_t ldd) {
    __shared__ uint4 As[BM * kChunksPerRow];
    __shared__ uint4 Bs[BN * kChunksPerRow];
    // Grouped launch order: runs of 8 M-tiles sweep the N-tiles, so that
    // concurrently running workgroups share A and B tiles in L2.
    const int64_t tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    const int64_t pid = blockIdx.x;
    constexpr int64_t G = 8;
    const int64_t group = pid / (G * tiles_n);
    const int64_t first_m = group * G;
    const int64_t gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
    const int64_t pm = first_m + (pid % (G * tiles_n)) % gsize;
    const int64_t pn = (pid % (G * tiles_n)) / gsize;
    const int64_t row0 = pm * BM, col0 = pn * BN;

    TileArgs t{a + row0 * lda, b + col0 * ldb, lda, ldb, m - row0, n - col0, k};
    v16f acc[2][2];
    mma_tile<FA, FB>(t, acc, As, Bs);
    store_tile_out<OUT_F32>(acc, d, ldd, row0, m - row0, col0, n - col0, sa, sa_vec, sb, sb_vec);
}

// Grouped: the linear workgroup index enumerates, group by group, the
// (m-tile, n-tile) pairs of each expert's row range. Each workgroup finds its
// group by walking the device offsets (the grid is an upper bound computed on
// the host without reading them: sum_g ceil(m_g/BM) <= ceil(total/BM) + G);
// workgroups past the last tile exit.
template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_grouped_gemm(const uint8_t* __restrict__ a, int64_t lda,
                                                           const uint8_t* __restrict__ b, int64_t ldb,
                                                           int64_t b_group_stride, const int64_t* __restrict__ offsets,
                                                           int g, int64_t total_m, int64_t n, int64_t k,
                                                           const float* __restrict__ sa, const float* __restrict__ sb,
                                                           void* __restrict__ d, int64_t ldd) {
    __shared__ uint4 As[BM * kChunksPerRow];
    __shared__ uint4 Bs[BN * kChunksPerRow];
    const int64_t tiles_n = (n + BN - 1) / BN;
    int64_t pid = blockIdx.x;
    int grp = -1;
    int64_t lo = 0, hi = 0;
    for (int e = 0; e < g; ++e) {
        int64_t s = offsets[e], t = offsets[e + 1];
        s = s < 0 ? 0 : (s > total_m ? total_m : s);
        t = t < s ? s : (t > total_m ? total_m : t);
        const int64_t tiles = ((t - s + BM - 1) / BM) * tiles_n;
        if (pid < tiles) {
            grp = e;
            lo = s;
            hi = t;
            break;
        }
        pid -= tiles;
    }
    if (grp < 0) return;
    const int64_t pm = pid / tiles_n, pn = pid % tiles_n;
    const int64_t row0 = lo + pm * BM, col0 = pn * BN;
    const uint8_t* bg = b + (int64_t)grp * b_group_stride;
    TileArgs t{a + row0 * lda, bg + col0 * ldb, lda, ldb, hi - row0, n - col0, k};
    v16f acc[2][2];
    mma_tile<FA, FB>(t, acc, As, Bs);
    store_tile_out<OUT_F32>(acc, d, ldd, row0, hi - row0, col0, n - col0, sa, 1, sb + (int64_t)grp * n, 1);
}

// ---------------------------------------------------------------------------
// Compatibility path for fnuz operands ("FP8 Training on MI300X": the fnuz
// encodings e4m3fnuz / e5m2fnuz that MI300-generation parts consume; gfx950's
// matrix cores take only the OCP encodings, and no fixed re-encoding maps
// either fnuz format onto an OCP one: e4m3fnuz holds 2^-10 and, read as OCP
// bits, 240 is a NaN code). Every FP8 value of any of the four encodings is
// exactly a bf16 value (at most 4 significant bits, exponents within bf16's
// normal range), so the operands are decoded to bf16 through a 256-entry table
// in LDS and multiplied on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16):
// each product of two decoded values is exact in fp32 and the sum is an fp32
// accumulation, the arithmetic of the FP8 path. 128 x 128 tiles, 32-deep K
// steps staged as bf16 in LDS; a correctness path, not tuned.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// bf16 bit pattern of FP8 code c in encoding F (NaN codes -> quiet NaN, OCP
// e5m2 Inf -> Inf).
template <int F>
__device__ __forceinline__ uint32_t fp8_to_bf16_bits(uint32_t c) {
    using T = FmtTraits<F>;
    constexpr int mb = T::mbits, eb = 7 - mb;
    const uint32_t sign = (c & 0x80u) << 8;
    const uint32_t e = (c >> mb) & ((1u << eb) - 1u), m = c & ((1u << mb) - 1u);
    if (T::fnuz) {
        if (c == 0x80u) return 0x7fc0u;
    } else if (F == kE4M3) {
        if ((c & 0x7fu) == 0x7fu) return sign | 0x7fc0u;
    } else {
        if (e == 31u) return m == 0u ? (sign | 0x7f80u) : (sign | 0x7fc0u);
    }
    if (e == 0u) {
        if (m == 0u) return sign;                        // zero (OCP keeps the sign)
        const int p = 31 - __builtin_clz(m);             // leading one of the subnormal mantissa
        const uint32_t exp = (uint32_t)(p + 1 - T::bias - mb + 127);
        return sign | (exp << 7) | ((m - (1u << p)) << (7 - p));
    }
    return sign | ((e - (uint32_t)T::bias + 127u) << 7) | (m << (7 - mb));
}

template <int F>
__device__ __forceinline__ void fill_bf16_table(uint16_t* lut) {
    lut[threadIdx.x] = (uint16_t)fp8_to_bf16_bits<F>(threadIdx.x);    // (256 threads: one code each)
}

namespace compat {
constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kPitch = BK + 8;                           // bf16 per LDS row (80 bytes: spreads the fragment reads)
}  // namespace compat

// Loads 16 codes (row t / 2, K half t % 2 of the 32-deep step) of a 128-row
// operand tile, decodes them through lut and stores them as bf16 in LDS.
__device__ __forceinline__ void compat_stage(const uint8_t* base, int64_t ld, int64_t valid_rows, int64_t k0, int64_t k,
                                             const uint16_t* lut, uint16_t* lds) {
    const int t = threadIdx.x;
    const int row = t >> 1, kh = (t & 1) * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < valid_rows && k0 + kh < k)                 // (k % 16 == 0: a 16-code chunk is whole or absent)
        v = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld + k0 + kh);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t word = w[i >> 1] >> (16 * (i & 1));
        o[i] = (uint32_t)lut[word & 0xffu] | ((uint32_t)lut[(word >> 8) & 0xffu] << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(lds + row * compat::kPitch + kh);
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

// One 128 x 128 tile of d = a * b^T with bf16-decoded operands: wavefront w owns
// the 64 x 64 quarter (w / 2, w % 2) as 2 x 2 blocks of 32 x 32.
template <int FA, int FB>
__device__ __forceinline__ void compat_tile(const uint8_t* a, int64_t lda, int64_t a_rows, const uint8_t* b,
                                            int64_t ldb, int64_t b_rows, int64_t k, v16f (&acc)[2][2]) {
    __shared__ uint16_t lut_a[256], lut_b[256];
    __shared__ __attribute__((aligned(16))) uint16_t As[compat::BM * compat::kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[compat::BN * compat::kPitch];
    fill_bf16_table<FA>(lut_a);
    fill_bf16_table<FB>(lut_b);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    for (int64_t k0 = 0; k0 < k; k0 += compat::BK) {
        __syncthreads();                                 // the tables are written; the previous step's reads are done
        compat_stage(a, lda, a_rows, k0, k, lut_a, As);
        compat_stage(b, ldb, b_rows, k0, k, lut_b, Bs);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            // lane l: row l % 32 of its block, 8 consecutive K of the 16-deep slice kk
            // (the same map for a and b, so equal K indices are paired)
            const int kc = kk * 16 + (lane >> 5) * 8;
            v8bf fa[2], fb[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = *reinterpret_cast<const v8bf*>(As + (wm * 64 + mi * 32 + (lane & 31)) * compat::kPitch + kc);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                fb[ni] = *reinterpret_cast<const v8bf*>(Bs + (wn * 64 + ni * 32 + (lane & 31)) * compat::kPitch + kc);
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
        }
    }
}

template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_gemm_compat(const uint8_t* __restrict__ a, int64_t lda,
                                                          const uint8_t* __restrict__ b, int64_t ldb, int64_t m,
                                                          int64_t n, int64_t k, const float* __restrict__ sa,
                                                          int sa_vec, const float* __restrict__ sb, int sb_vec,
                                                          void* __restrict__ d, int64_t ldd) {
    const int64_t tiles_n = (n + compat::BN - 1) / compat::BN;
    const int64_t row0 = (int64_t)(blockIdx.x / tiles_n) * compat::BM, col0 = (int64_t)(blockIdx.x % tiles_n) * compat::BN;
    v16f acc[2][2];
    compat_tile<FA, FB>(a + row0 * lda, lda, m - row0, b + col0 * ldb, ldb, n - col0, k, acc);
    store_tile_out<OUT_F32>(acc, d, ldd, row0, m - row0, col0, n - col0, sa, sa_vec, sb, sb_vec);
}

// Grouped form: the linear workgroup index enumerates each group's (m-tile,
// n-tile) pairs group after group (as k_grouped_gemm).
template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_grouped_gemm_compat(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ b, int64_t ldb, int64_t b_group_stride,
    const int64_t* __restrict__ offsets, int g, int64_t total_m, int64_t n, int64_t k, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ d, int64_t ldd) {
    const int64_t tiles_n = (n + compat::BN - 1) / compat::BN;
    int64_t pid = blockIdx.x;
    int grp = -1;
    int64_t lo = 0, hi = 0;
    for (int e = 0; e < g; ++e) {
        int64_t s0 = offsets[e], s1 = offsets[e + 1];
        s0 = s0 < 0 ? 0 : (s0 > total_m ? total_m : s0);
        s1 = s1 < s0 ? s0 : (s1 > total_m ? total_m : s1);
        const int64_t tiles = ((s1 - s0 + compat::BM - 1) / compat::BM) * tiles_n;
        if (pid < tiles) {
            grp = e;
            lo = s0;
            hi = s1;
            break;
        }
        pid -= tiles;
    }
    if (grp < 0) return;
    const int64_t row0 = lo + (pid / tiles_n) * compat::BM, col0 = (pid % tiles_n) * compat::BN;
    const uint8_t* bg = b + (int64_t)grp * b_group_stride;
    v16f acc[2][2];
    compat_tile<FA, FB>(a + row0 * lda, lda, hi - row0, bg + col0 * ldb, ldb, n - col0, k, acc);
    store_tile_out<OUT_F32>(acc, d, ldd, row0, hi - row0, col0, n - col0, sa, 1, sb + (int64_t)grp * n, 1);
}

// ---------------------------------------------------------------------------
// Large-tile kernels: 256 x 256 output tile per workgroup, one 128 x 128
// quadrant per wavefront (4 x 4 blocks of 32x32x64, 256 fp32 accumulators per
// lane in AGPRs). The K loop (k128_mainloop below) streams the operands through
// LDS with direct global->LDS loads issued from inline assembly: the compiler
// cannot see that they write LDS, so it adds no waits of its own; explicit
// vmcnt waits at the right points do. Rows past m / n are clamped to the last
// valid row on load and never stored. Requires k % 256 == 0.
namespace big {
constexpr int BM = 256, BN = 256;
constexpr int kEpiWave = 32 * 1024;                 // one wavefront's staged 128 x 128 bf16 block
constexpr int kMain = 4 * kEpiWave;                 // 128 KB: two K stages, or the staged output
constexpr int kScaleOff = kMain;                    // 256 row scales, then 256 column scales (fp32)
constexpr int kSmem = kMain + 2 * 256 * 4;
// MX operands: per K step, each of the 256 A rows and 256 B rows brings one
// dword of E8M0 block scales (its four 32-element blocks), in two stages
constexpr int kMxStage = 2 * 256 * 4;
constexpr int kMxOff = kSmem;
constexpr int kSmemMx = kSmem + 2 * kMxStage;       // 134 KB
}  // namespace big

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait for vmcnt <= N (and lgkmcnt <= L), leave expcnt alone.
template <int N, int L = 15>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64 && L >= 0 && L < 16, "counter range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070 | (L << 8));
}

// One direct global->LDS load of 16 bytes per lane: lane l's bytes land at
// LDS address lds_base + 16 l (lds_base wave-uniform, set through M0; one
// wait state between the M0 write and the load). M0 is clobbered: the kernels
// that use this have no other M0 user (the build's ISA check test asserts it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(uint32_t lds_base, const uint8_t* gptr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}
// The same load with the address split into a wave-uniform 64-bit base
// (SGPRs) and the lane's 32-bit byte offset (the instruction's SGPR-base
// form: one VGPR per lane instead of two). The base's halves go through
// v_readfirstlane, whose result is a signed int: each half is zero-extended
// before the two are joined (a sign-extended low half would set every bit of
// the high half for an address whose bit 31 is set). The s_nop gives the five
// wait states that a VMEM instruction reading an SGPR needs after a VALU
// instruction (such as v_readfirstlane) wrote it; the compiler does not
// account for the SGPR reads of an asm statement.
__device__ __forceinline__ void lds_dma16_s(uint32_t lds_base, const uint8_t* base, uint32_t voff) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t hi = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    const uint64_t lo = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_base), "v"(voff), "s"((hi << 32) | lo)
                 : "memory", "m0");
}
// Same with 4 bytes per lane: lane l's dword lands at lds_base + 4 l.
__device__ __forceinline__ void lds_dma4(uint32_t lds_base, const void* gptr) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds_base), "v"(gptr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ int big_row(int j) {   // j < 4: A block j; j >= 4: B block j-4 (row in its tile)
    const int w = threadIdx.x >> 6;
    return (j < 4 ? (w >> 1) * 128 + j * 32 : (w & 1) * 128 + (j - 4) * 32) + (threadIdx.x & 31);
}
__device__ __forceinline__ v8i big_join(u32x4 lo, u32x4 hi) {
    v8i f;
    f[0] = (int)lo[0]; f[1] = (int)lo[1]; f[2] = (int)lo[2]; f[3] = (int)lo[3];
    f[4] = (int)hi[0]; f[5] = (int)hi[1]; f[6] = (int)hi[2]; f[7] = (int)hi[3];
    return f;
}

// Logical tile of workgroup `bid` among `nt` tiles: the hardware deals
// workgroups to the 8 XCDs round-robin, so each XCD's share is mapped to a
// contiguous run of logical tiles (neighbouring tiles share A/B panels in that
// XCD's L2); within the run, groups of `gm` M-tiles sweep the N-tiles.
__device__ __forceinline__ void big_tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t* pm,
                                                int64_t* pn) {
    const int64_t nt = tiles_m * tiles_n;
    const int64_t q = nt / 8, rem = nt % 8;
    const int64_t xcd = bid % 8, idx = bid / 8;
    const int64_t t = xcd * q + (xcd < rem ? xcd : rem) + idx;
    constexpr int64_t gm = 4;
    const int64_t group = t / (gm * tiles_n);
    const int64_t first_m = group * gm;
    const int64_t gsize = tiles_m - first_m < gm ? tiles_m - first_m : gm;
    *pm = first_m + (t % (gm * tiles_n)) % gsize;
    *pn = (t % (gm * tiles_n)) / gsize;
}

// MX block scales of a step in LDS: row r of the tile (A, then B at +1 KB) at
// dword (r / 128) * 128 + (r % 32) * 4 + (r / 32) % 4, so the four rows
// wm*128 + 32 mi + l (mi = 0..3) that lane l needs are one 16-byte read. The
// thread that fills dword i (a wavefront's direct load fills 64 consecutive
// dwords) loads row mx_row(i).
__device__ __forceinline__ int mx_row(int i) { return (i >> 7) * 128 + (i & 3) * 32 + ((i & 127) >> 2); }

// The four scale dwords of lane l's rows, shifted by the lane half s = l / 32:
// lane half s supplies the scale of block s of each 64-deep half, so byte 0 is
// then block s of the step's first half and byte 2 block s of its second.
__device__ __forceinline__ u32x4 mx_scales(const uint8_t* stage, int half_sel) {
    const int lane = threadIdx.x & 63;
    const int w = (threadIdx.x >> 6);
    const int base = half_sel == 0 ? (w >> 1) * 128 : 256 + (w & 1) * 128;
    u32x4 v = *reinterpret_cast<const u32x4*>(stage + 4 * (base + (lane & 31) * 4));
    const int sh = 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] >>= sh;
    return v;
}

// MFMA of one 64-deep half: with MX the E8M0 scale bytes OPSEL of the lane's
// A and B scale dwords, else unscaled.
template <int FA, int FB, bool MX, int OPSEL>
__device__ __forceinline__ v16f mfma64(const v8i& fa, const v8i& fb, const v16f& c, uint32_t xa, uint32_t xb) {
    if constexpr (MX)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, c, MfmaFmt<FA>::v, MfmaFmt<FB>::v, OPSEL,
                                                               (int)xa, OPSEL, (int)xb);
    else
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa, fb, c, MfmaFmt<FA>::v, MfmaFmt<FB>::v, 0, 0, 0, 0);
}

// K128 main loop of the large-tile kernels: K advances 128 bytes per step
// through two 64 KB LDS stages (A: 256 rows x 128 B, then B). Each direct load
// brings whole 128-byte row segments (8 lanes per row), so the L1 sends
// full-line requests to L2: on gfx950 the load path's throughput goes with the
// number of requests (a loop of 64-deep steps, whose loads move 64-byte row
// segments, was ~13% slower at these shapes). With two stages the loads of step p+2 are
// issued during the second half of step p and waited for in the middle of
// step p+1 (a barrier between the two halves of each step); step p's
// second-half fragments are read during its first 16 MFMAs and step p+1's
// first-half fragments during its last 16. 128-byte rows: chunk c of row r sits in slot c ^ ((r >> 1) & 7),
// so 16 consecutive rows reading one chunk hit 16 distinct 16-byte bank groups.
namespace k128 {
constexpr int BK = 128;
constexpr int kOpBytes = 256 * BK;                   // one operand of a stage: 32 KB
constexpr int kStage = 2 * kOpBytes;                 // 64 KB
static_assert(2 * kStage == big::kScaleOff, "two stages below the scale area");
}  // namespace k128

__device__ __forceinline__ int k128_slot(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Per-lane byte offsets of this thread's 8 loads of one operand: load i of
// wavefront w fills rows w*64 + 8i .. w*64 + 8i + 7 (1 KB, 16 bytes per lane):
// lane l takes row + l / 8, slot l % 8, i.e. the chunk stored in that slot.
// 32-bit arithmetic (ld < 2^24); rows past the last valid one are clamped.
__device__ __forceinline__ void k128_lane_offsets(uint32_t (&off)[8], int64_t ld, int64_t valid_rows) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t ld32 = (uint32_t)ld;
    const int last = (int)(valid_rows < 256 ? valid_rows : 256) - 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = wave * 64 + i * 8 + (lane >> 3);
        const int chunk = k128_slot(row, lane & 7);     // the slot map is an involution
        const uint32_t r = (uint32_t)(row < last ? row : last);
        off[i] = r * ld32 + (uint32_t)(chunk * 16);
    }
}

// Fragment half of the 32x32x64 instruction for K half h (bytes 64h ..
// 64h + 63 of the 128-byte row), in two 16-byte pieces hh. The instruction's
// own K order: lane half s = lane / 32 holds K 16s .. 16s + 15 in its bytes
// 0-15 and K 32 + 16s .. 32 + 16s + 15 in bytes 16-31, and with block scales
// the scale of lane half s covers K 32s .. 32s + 31, i.e. bytes 0-15 of both
// lane halves form the first 32-element block (measured on gfx950). That
// order is taken with MX. Without block scales any order common to A and B
// gives the same sums, and lane half s takes bytes 32s .. 32s + 31.
template <bool MX>
__device__ __forceinline__ u32x4 k128_half(const uint8_t* tile, int row, int h, int hh) {
    const int s = (threadIdx.x & 63) >> 5;
    const int c = MX ? h * 4 + s + 2 * hh : h * 4 + s * 2 + hh;
    return *reinterpret_cast<const u32x4*>(tile + row * 128 + (k128_slot(row, c) << 4));
}

// Fragment order of a step: A0, B0, B1, B2, B3, A1, A2, A3 (the order the MFMA
// sweep (mi, ni) = (0,0), (0,1), .. first needs them). j < 4: A block j, else B.
__device__ __forceinline__ int k128_frag(int f) { return f == 0 ? 0 : (f <= 4 ? 4 + (f - 1) : f - 4); }

// Step p with stage CUR = p % 2 (compile-time). On entry f0 holds step p's
// first-half fragments and sx its A and B scale dwords (MX), both read during
// step p-1 (or the prologue). The step:
//   16 MFMAs on f0, each followed by one read of step p's second-half
//   fragments from stage CUR
//   wait until this thread's loads have landed (those of step p+1, issued
//   during step p-1); barrier: stage CUR^1 is complete and every wavefront
//   has read stage CUR for the last time
//   16 MFMAs on f1, each followed (NEXT) by one read of step p+1's first-half
//   fragments from stage CUR^1 and (LOADS) by one of the 16 loads of step p+2
//   (K offset knext) into stage CUR; with MX also step p+2's two scale dwords
//   per thread (the records xa / xb of K step 0 advanced by knext / 128 steps
//   of xsa / xsb bytes), and step p+1's scales read into sx.
// A step's MFMAs thus never wait for LDS reads issued after the barrier, and
// the loads have a full step to land. With issue false (uniform) a LOADS step
// skips its loads: the same code, so a K loop whose last pair loads nothing
// needs no second copy of the steps. With ZERO the first 16 MFMAs start from
// zero instead of acc (a tile's first step: no zeroing pass). SADDR: the loads
// take the SGPR-base form (a, b wave-uniform bases, aoff / boff lane offsets).
template <int FA, int FB, int CUR, bool NEXT, bool LOADS, bool MX, bool SADDR = false, bool ZERO = false>
__device__ __forceinline__ void k128_step(uint8_t* smem, v16f (&acc)[4][4], v8i (&f0)[8], u32x4 (&sx)[2],
                                          const uint8_t* a, const uint32_t (&aoff)[8], const uint8_t* b,
                                          const uint32_t (&boff)[8], int64_t knext, const uint8_t* xa,
                                          const uint8_t* xb, int64_t xsa, int64_t xsb, bool issue = true) {
    const uint8_t* ta = smem + CUR * k128::kStage;
    const uint8_t* tb = ta + k128::kOpBytes;
    const uint8_t* na = smem + (CUR ^ 1) * k128::kStage;
    const uint8_t* nb = na + k128::kOpBytes;
    u32x4 h1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int mi = i >> 2, ni = i & 3;
        acc[mi][ni] = mfma64<FA, FB, MX, 0>(f0[mi], f0[4 + ni], ZERO ? v16f{} : acc[mi][ni], sx[0][mi], sx[1][ni]);
        const int j = k128_frag(i >> 1);
        h1[i] = k128_half<MX>(j < 4 ? ta : tb, big_row(j), 1, i & 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    v8i f1[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) f1[k128_frag(f)] = big_join(h1[2 * f], h1[2 * f + 1]);
    wait_vmcnt<0, 0>();
    __syncthreads();
    const u32x4 sxc[2] = {sx[0], sx[1]};
    if constexpr (MX && NEXT) {
        const uint8_t* xs = smem + big::kMxOff + (CUR ^ 1) * big::kMxStage;
        sx[0] = mx_scales(xs, 0);
        sx[1] = mx_scales(xs, 1);
    }
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t dma_base = __builtin_amdgcn_readfirstlane(lds_addr(smem + CUR * k128::kStage)) + wave * 8192;
    u32x4 h0[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int mi = i >> 2, ni = i & 3;
        acc[mi][ni] = mfma64<FA, FB, MX, 2>(f1[mi], f1[4 + ni], acc[mi][ni], sxc[0][mi], sxc[1][ni]);
        if (NEXT) {
            const int j = k128_frag(i >> 1);
            h0[i] = k128_half<MX>(j < 4 ? na : nb, big_row(j), 0, i & 1);
        }
        if (LOADS && issue) {
            if constexpr (SADDR) {
                if (i < 8)
                    lds_dma16_s(dma_base + i * 1024, a + knext, aoff[i]);
                else
                    lds_dma16_s(dma_base + k128::kOpBytes + (i - 8) * 1024, b + knext, boff[i - 8]);
            } else {
                if (i < 8)
                    lds_dma16(dma_base + i * 1024, a + knext + aoff[i]);
                else
                    lds_dma16(dma_base + k128::kOpBytes + (i - 8) * 1024, b + knext + boff[i - 8]);
            }
            if constexpr (MX) {
                if (i == 3 || i == 11) {
                    const uint32_t xbase = __builtin_amdgcn_readfirstlane(
                                               lds_addr(smem + big::kMxOff + CUR * big::kMxStage)) +
                                           wave * 256 + (i == 3 ? 0 : 1024);
                    lds_dma4(xbase, i == 3 ? xa + (knext / k128::BK) * xsa : xb + (knext / k128::BK) * xsb);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) {
#pragma unroll
        for (int f = 0; f < 8; ++f) f0[k128_frag(f)] = big_join(h0[2 * f], h0[2 * f + 1]);
    }
}

// The K loop of the large-tile kernels; k % 256 == 0, k > 0. The
// epilogue's row and column scales go to the scale area: sa_lane / sb_lane
// (thread t's row / column scale) or, with MX, 1 (the block scales are applied
// inside the MFMAs; xa / xb are the K-step-0 scale records of A row mx_row(t)
// and B row mx_row(t) of the tile, and a K step advances them by xsa / xsb
// bytes). Prologue: steps 0 and 1 in flight, wait for step 0, read its
// first-half fragments.
template <int FA, int FB, bool MX>
__device__ __forceinline__ void k128_mainloop(uint8_t* smem, const uint8_t* a, int64_t lda, int64_t a_rows,
                                              const uint8_t* b, int64_t ldb, int64_t b_rows, int64_t k,
                                              const float* sa_lane, const float* sb_lane, const uint8_t* xa,
                                              const uint8_t* xb, int64_t xsa, int64_t xsb, v16f (&acc)[4][4]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    uint32_t aoff[8], boff[8];
    k128_lane_offsets(aoff, lda, a_rows);
    k128_lane_offsets(boff, ldb, b_rows);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nk = k / k128::BK;
    constexpr int L = MX ? 18 : 16;                      // loads per thread per step
    v8i f0[8];
    u32x4 sx[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    {
        if constexpr (MX) {
            float* s = reinterpret_cast<float*>(smem + big::kScaleOff);
            s[threadIdx.x] = 1.0f;
            s[256 + threadIdx.x] = 1.0f;
        } else {
            const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kScaleOff)) + wave * 256;
            lds_dma4(sbase, sa_lane);
            lds_dma4(sbase + 1024, sb_lane);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * k128::kStage)) + wave * 8192;
            const int64_t k0 = s * k128::BK;
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_dma16(base + i * 1024, a + k0 + aoff[i]);
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_dma16(base + k128::kOpBytes + i * 1024, b + k0 + boff[i]);
            if constexpr (MX) {
                const uint32_t xbase =
                    __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kMxOff + s * big::kMxStage)) + wave * 256;
                lds_dma4(xbase, xa + s * xsa);
                lds_dma4(xbase + 1024, xb + s * xsb);
            }
        }
        wait_vmcnt<L>();                                 // step 0 (and the scales) landed
        __syncthreads();
#pragma unroll
        for (int f = 0; f < 8; ++f) {
            const int j = k128_frag(f);
            f0[j] = big_join(k128_half<MX>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 0),
                             k128_half<MX>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 1));
        }
        if constexpr (MX) {
            sx[0] = mx_scales(smem + big::kMxOff, 0);
            sx[1] = mx_scales(smem + big::kMxOff, 1);
        }
    }
    // one loop over the step pairs: one path, so the sums keep one register
    // assignment from the zeroing to the epilogue. The last pair issues no
    // loads; with MX it loads the tile's steps 0 and 1 again instead (valid
    // addresses, never read: skipping the loads there costs registers)
    int64_t p = 0;
    do {                                                 // nk >= 2
        const bool more = p + 2 < nk;
        const int64_t kl = more ? (p + 2) * k128::BK : 0;
        k128_step<FA, FB, 0, true, true, MX>(smem, acc, f0, sx, a, aoff, b, boff, kl, xa, xb, xsa, xsb, more || MX);
        k128_step<FA, FB, 1, true, true, MX>(smem, acc, f0, sx, a, aoff, b, boff, kl + k128::BK, xa, xb, xsa, xsb,
                                             more || MX);
        p += 2;
    } while (p < nk);
    wait_vmcnt<0>();                                     // (MX: the last pair's loads landed)
}

// Staged bf16 block of the epilogue: group g of 4 rows, column c -> 8 bytes
// (the 4 rows' values) at g * 1024 + unit * 16 + (c % 2) * 8, where the 16-byte
// unit c / 2 = u is stored at (u & ~3) | ((u ^ (u >> 4)) & 3): the 16 lanes of
// one 16-byte read (units 4i + k, i = 0..15) then hit 16 distinct bank groups,
// and the 32 lanes of one 8-byte write still cover 256 contiguous bytes.
__device__ __forceinline__ int epi_off(int g, int c) {
    const int u = c >> 1;
    return g * 1024 + (((u & ~3) | ((u ^ (u >> 4)) & 3)) << 4) + ((c & 1) << 3);
}

// Epilogue of a 256 x 256 tile at (row0, col0) with rows_total / cols_total
// valid rows / columns from there: d = acc * sa_row * sb_col, the 256 row and
// 256 column scales of the tile sitting in the scale area of LDS.
template <bool OUT_F32>
__device__ __forceinline__ void big_epilogue(uint8_t* smem, v16f (&acc)[4][4], void* __restrict__ d,
                                             int64_t ldd, int64_t row0, int64_t rows_total, int64_t col0,
                                             int64_t cols_total, int vec_out) {
    // The thread index is made opaque here, so the epilogue's lane arithmetic
    // is not hoisted above the main loop (where it would stay live and spill).
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t wrow0 = row0 + wm * 128, wcol0 = col0 + wn * 128;
    const int64_t rows_valid = rows_total - wm * 128, cols_valid = cols_total - wn * 128;
    // The accumulators stay in AGPRs until each is used: without this the
    // compiler copies all 256 to VGPRs at once at the end of the loop and spills.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    // every wavefront is done with the stages (the staging below reuses them),
    // and every lane's scale load has landed (the main loop ends with vmcnt 0)
    __syncthreads();
    const float* s_rows = reinterpret_cast<const float*>(smem + big::kScaleOff);
    const float* s_cols = s_rows + 256;
    float sbj[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) sbj[ni] = s_cols[wn * 128 + ni * 32 + (lane & 31)];
    if (OUT_F32) {
        // direct stores from registers
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (lr >= rows_valid) continue;
                const float sai = s_rows[wm * 128 + lr];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int lc = ni * 32 + (lane & 31);
                    if (lc >= cols_valid) continue;
                    const float v = acc[mi][ni][r] * sai * sbj[ni];
                    const int64_t off = (wrow0 + lr) * ldd + wcol0 + lc;
                    reinterpret_cast<float*>(d)[off] = v;
                }
            }
        return;
    }
    // bf16 through LDS, each wavefront on its own 128 x 128 block (no barrier
    // between writing and reading it back: a wavefront's LDS operations are
    // done in order). A lane's registers hold 4 consecutive rows of one column
    // (acc[mi][ni][4q .. 4q+3]); they go out as one 8-byte write per column.
    // The read-back takes 8 columns x 4 rows per lane (four 16-byte reads) and
    // byte-permutes them into four row chunks of 8 columns: 16-byte stores, 16
    // lanes per 256 contiguous bytes of a row, marked nontemporal (the output is
    // not read again here, and streaming it leaves the caches to the operand
    // panels: 0.5-1% faster at the Llama3-8B shapes).
    uint8_t* ep = smem + wave * big::kEpiWave;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int g = 8 * mi + 2 * q + (lane >> 5);              // rows 4g .. 4g+3 of the block
            const u32x4 s4 = *reinterpret_cast<const u32x4*>(&s_rows[wm * 128 + 4 * g]);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int r = 4 * q;
                v2f v01 = {acc[mi][ni][r] * __uint_as_float(s4[0]) * sbj[ni],
                           acc[mi][ni][r + 1] * __uint_as_float(s4[1]) * sbj[ni]};
                v2f v23 = {acc[mi][ni][r + 2] * __uint_as_float(s4[2]) * sbj[ni],
                           acc[mi][ni][r + 3] * __uint_as_float(s4[3]) * sbj[ni]};
                uint2 w;
                w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, v2bf));
                w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, v2bf));
                *reinterpret_cast<uint2*>(ep + epi_off(g, 32 * ni + (lane & 31))) = w;
            }
        }
    wait_vmcnt<63, 0>();                                 // this wavefront's staging writes are done
    __builtin_amdgcn_wave_barrier();
    const int cc = lane & 15;                            // columns 8cc .. 8cc+7
    const bool full_cols = vec_out && 8 * cc + 8 <= cols_valid;
#pragma unroll 2
    for (int it = 0; it < 8; ++it) {
        const int g = 4 * it + (lane >> 4);
        u32x4 un[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) un[k] = *reinterpret_cast<const u32x4*>(ep + epi_off(g, 8 * cc + 2 * k));
        // unit k: column 8cc+2k in words 0 (rows 0, 1) and 1 (rows 2, 3), column 8cc+2k+1 in words 2 and 3
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lr = 4 * g + r;
            if (lr >= rows_valid) continue;
            const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
            const int wlo = (r >> 1), whi = 2 + (r >> 1);
            u32x4 row;
#pragma unroll
            for (int k = 0; k < 4; ++k) row[k] = __builtin_amdgcn_perm(un[k][whi], un[k][wlo], sel);
            uint16_t* dst = reinterpret_cast<uint16_t*>(d) + (wrow0 + lr) * ldd + wcol0 + 8 * cc;
            if (full_cols) {
                __builtin_nontemporal_store(row, reinterpret_cast<u32x4*>(dst));
            } else {
                for (int e = 0; e < 8 && 8 * cc + e < cols_valid; ++e)
                    dst[e] = (uint16_t)(row[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_big(const uint8_t* __restrict__ a, int64_t lda,
                                                     const uint8_t* __restrict__ b, int64_t ldb, int64_t m, int64_t n,
                                                     int64_t k, const float* __restrict__ sa, int sa_vec,
                                                     const float* __restrict__ sb, int sb_vec, void* __restrict__ d,
                                                     int64_t ldd, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[big::kSmem];
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    int64_t pm, pn;
    big_tile_coords(blockIdx.x, tiles_m, tiles_n, &pm, &pn);
    const int64_t row0 = pm * big::BM, col0 = pn * big::BN;
    const int t = threadIdx.x;
    const float* sa_lane = sa + (sa_vec ? (row0 + t < m ? row0 + t : m - 1) : 0);
    const float* sb_lane = sb + (sb_vec ? (col0 + t < n ? col0 + t : n - 1) : 0);
    v16f acc[4][4];
    k128_mainloop<FA, FB, false>(smem, a + row0 * lda, lda, m - row0, b + col0 * ldb, ldb, n - col0, k, sa_lane,
                                 sb_lane, nullptr, nullptr, 0, 0, acc);
    big_epilogue<OUT_F32>(smem, acc, d, ldd, row0, m - row0, col0, n - col0, vec_out);
}

// An MX tile with k = 0: zero sums, unit scales (the K loop needs k > 0).
template <bool OUT_F32>
__device__ __forceinline__ void mx_zero_tile(uint8_t* smem, void* __restrict__ d, int64_t ldd, int64_t row0,
                                             int64_t rows, int64_t col0, int64_t cols, int vec_out) {
    float* s = reinterpret_cast<float*>(smem + big::kScaleOff);
    s[threadIdx.x] = 1.0f;                               // (the epilogue's barrier orders the scale area)
    s[256 + threadIdx.x] = 1.0f;
    v16f acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    big_epilogue<OUT_F32>(smem, acc, d, ldd, row0, rows, col0, cols, vec_out);
}

// MX product: d = sum over 32-deep K blocks of the blocks' dot products times
// 2^(xa - 127) * 2^(xb - 127), the E8M0 scales of row i's and column j's block
// (K-step-major records: the scales of blocks 4j .. 4j+3 of row r are the
// 4 bytes at xa + 4 (j ld_xa + r)).
template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_gemm_mx(const uint8_t* __restrict__ a, int64_t lda,
                                                    const uint8_t* __restrict__ xa, int64_t ld_xa,
                                                    const uint8_t* __restrict__ b, int64_t ldb,
                                                    const uint8_t* __restrict__ xb, int64_t ld_xb, int64_t m, int64_t n,
                                                    int64_t k, void* __restrict__ d, int64_t ldd, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[big::kSmemMx];
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    int64_t pm, pn;
    big_tile_coords(blockIdx.x, tiles_m, tiles_n, &pm, &pn);
    const int64_t row0 = pm * big::BM, col0 = pn * big::BN;
    const int rt = mx_row(threadIdx.x);
    const uint8_t* xa_lane = xa + 4 * (row0 + rt < m ? row0 + rt : m - 1);
    const uint8_t* xb_lane = xb + 4 * (col0 + rt < n ? col0 + rt : n - 1);
    if (k == 0) {
        mx_zero_tile<OUT_F32>(smem, d, ldd, row0, m - row0, col0, n - col0, vec_out);
        return;
    }
    v16f acc[4][4];
    k128_mainloop<FA, FB, true>(smem, a + row0 * lda, lda, m - row0, b + col0 * ldb, ldb, n - col0, k, nullptr,
                                nullptr, xa_lane, xb_lane, 4 * ld_xa, 4 * ld_xb, acc);
    big_epilogue<OUT_F32>(smem, acc, d, ldd, row0, m - row0, col0, n - col0, vec_out);
}

// Grouped large-tile kernel. Group e owns rows lo_e .. hi_e of a and d (the
// offsets clamped to [0, total_m], hi_e >= lo_e) and the n x k matrix
// b + e * b_group_stride; its tiles are the ceil((hi_e - lo_e) / 256) x
// ceil(n / 256) tiles of that row range. The grid is an upper bound computed
// on the host without reading the offsets (sum_e ceil(m_e / 256) <=
// ceil(total / 256) + g). Each workgroup builds the exclusive prefix sum of the
// per-group tile counts in LDS (256 threads, g / 256 groups each, then a block
// scan), so it knows the real tile count nt: workgroups at or past nt exit (they
// are dispatched last); the others take the XCD-aware order of the dense
// kernel over the concatenated per-group tile lists (a run of workgroups on one
// XCD covers neighbouring tiles of one group: shared b panels and a rows in
// that XCD's L2) and find their group by binary search in the prefix sums.
constexpr int kMaxGroupsBig = 4096;
static_assert((kMaxGroupsBig + 1) * 8 <= big::kMain, "group prefix sums fit in the stage buffers");

// With MX the operands carry E8M0 block scales instead of sa / sb: xa (row r
// of a in the records of xa with ld_xa) and, for group e, xb + e *
// xb_group_stride (bytes) with ld_xb.
template <int FA, int FB, bool OUT_F32, bool MX>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_big(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ b, int64_t ldb, int64_t b_group_stride,
    const int64_t* __restrict__ offsets, int g, int64_t total_m, int64_t n, int64_t k, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ d, int64_t ldd, int vec_out, const uint8_t* __restrict__ xa,
    int64_t ld_xa, const uint8_t* __restrict__ xb, int64_t ld_xb, int64_t xb_group_stride) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[MX ? big::kSmemMx : big::kSmem];
    const int64_t tiles_n = (n + big::BN - 1) / big::BN;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    auto bounds = [&](int e, int64_t* lo, int64_t* hi) {
        int64_t s = offsets[e], u = offsets[e + 1];
        s = s < 0 ? 0 : (s > total_m ? total_m : s);
        u = u < s ? s : (u > total_m ? total_m : u);
        *lo = s;
        *hi = u;
    };
    auto tiles_of = [&](int e) {
        int64_t lo, hi;
        bounds(e, &lo, &hi);
        return ((hi - lo + big::BM - 1) / big::BM) * tiles_n;
    };
    int64_t* pre = reinterpret_cast<int64_t*>(smem);                       // g + 1 prefix sums
    int64_t* wsum = reinterpret_cast<int64_t*>(smem + big::kScaleOff);     // 4 wavefront totals
    const int per = (g + 255) / 256;
    const int e0 = t * per, e1 = e0 + per < g ? e0 + per : g;
    int64_t mine = 0;
    for (int e = e0; e < e1; ++e) mine += tiles_of(e);
    int64_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int64_t run = incl - mine;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int e = e0; e < e1; ++e) {
        pre[e] = run;
        run += tiles_of(e);
    }
    if (t == 255) pre[g] = run;
    __syncthreads();
    const int64_t nt = pre[g];
    const int64_t bid = blockIdx.x;
    if (bid >= nt) return;                               // uniform over the workgroup
    const int64_t q = nt / 8, rem = nt % 8;
    const int64_t xcd = bid % 8, idx = bid / 8;
    int64_t lt = xcd * q + (xcd < rem ? xcd : rem) + idx;     // logical tile, < nt
    // last group e with pre[e] <= lt: a non-empty group (an empty one has pre[e+1] == pre[e])
    int lo_e = 0, hi_e = g;                              // pre[lo_e] <= lt < pre[hi_e]
    while (hi_e - lo_e > 1) {
        const int mid = (lo_e + hi_e) >> 1;
        if (pre[mid] <= lt)
            lo_e = mid;
        else
            hi_e = mid;
    }
    const int grp = lo_e;
    lt -= pre[grp];
    __syncthreads();                                     // the prefix sums are dead: the stages reuse LDS
    int64_t lo, hi;
    bounds(grp, &lo, &hi);
    // within the group: runs of 4 m-tiles sweep the n-tiles
    const int64_t tiles_m = (hi - lo + big::BM - 1) / big::BM;
    constexpr int64_t gm = 4;
    const int64_t first_m = (lt / (gm * tiles_n)) * gm;
    const int64_t gsize = tiles_m - first_m < gm ? tiles_m - first_m : gm;
    const int64_t pm = first_m + (lt % (gm * tiles_n)) % gsize;
    const int64_t pn = (lt % (gm * tiles_n)) / gsize;
    const int64_t row0 = lo + pm * big::BM, col0 = pn * big::BN;
    const uint8_t* bg = b + (int64_t)grp * b_group_stride;
    if (MX && k == 0) {
        mx_zero_tile<OUT_F32>(smem, d, ldd, row0, hi - row0, col0, n - col0, vec_out);
        return;
    }
    v16f acc[4][4];
    if constexpr (MX) {
        const int rt = mx_row(t);
        const uint8_t* xa_lane = xa + 4 * (row0 + rt < hi ? row0 + rt : hi - 1);
        const uint8_t* xb_lane = xb + (int64_t)grp * xb_group_stride + 4 * (col0 + rt < n ? col0 + rt : n - 1);
        k128_mainloop<FA, FB, true>(smem, a + row0 * lda, lda, hi - row0, bg + col0 * ldb, ldb, n - col0, k, nullptr,
                                    nullptr, xa_lane, xb_lane, 4 * ld_xa, 4 * ld_xb, acc);
    } else {
        const float* sa_lane = sa + (row0 + t < hi ? row0 + t : hi - 1);
        const float* sb_lane = sb + (int64_t)grp * n + (col0 + t < n ? col0 + t : n - 1);
        k128_mainloop<FA, FB, false>(smem, a + row0 * lda, lda, hi - row0, bg + col0 * ldb, ldb, n - col0, k, sa_lane,
                                     sb_lane, nullptr, nullptr, 0, 0, acc);
    }
    big_epilogue<OUT_F32>(smem, acc, d, ldd, row0, hi - row0, col0, n - col0, vec_out);
}

// Grouped product over ragged contraction ranges (the MoE weight gradient):
// D_g = A[:, P_g : P_g + K_g] B[:, P_g : P_g + K_g]^T * sa_g * sb_g with
// K_g = roundup(m_g, 256) over the grouped transposed layout (its zero padding
// adds nothing) and P_g the sum of the earlier groups' K_h. The grid holds
// G x per8 slots, per8 = tiles_m * tiles_n rounded up to 8: group g's tiles are
// dealt evenly to the 8 XCDs (slot w goes to XCD w % 8), contiguous within an
// XCD, so groups of very different K_g keep the XCDs balanced; slots past a
// group's tile count exit. Contraction columns at or past min(lda, ldb) are
// never read: a group whose padded range reaches them writes NaN.
template <int FA, int FB, bool OUT_F32>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_ragged_k(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ b, int64_t ldb,
    const int64_t* __restrict__ offsets, int G, int64_t total, int64_t m, int64_t n, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ d, int64_t ldd, int64_t d_group_stride, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[big::kSmem];
    __shared__ int64_t wsum[4];
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    const int64_t per = tiles_m * tiles_n, per8 = (per + 7) / 8 * 8;
    const int grp = (int)(blockIdx.x / per8);
    const int64_t wp = blockIdx.x % per8;
    const int64_t xcd = wp % 8, idx = wp / 8, q = per / 8, rem = per % 8;
    if (idx >= q + (xcd < rem ? 1 : 0)) return;        // uniform over the workgroup
    const int64_t lt = xcd * q + (xcd < rem ? xcd : rem) + idx;
    constexpr int64_t gm = 4;
    const int64_t first_m = (lt / (gm * tiles_n)) * gm;
    const int64_t gsize = tiles_m - first_m < gm ? tiles_m - first_m : gm;
    const int64_t pm = first_m + (lt % (gm * tiles_n)) % gsize;
    const int64_t pn = (lt % (gm * tiles_n)) / gsize;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    auto kpad = [&](int h) {
        int64_t lo = offsets[h], hi = offsets[h + 1];
        lo = lo < 0 ? 0 : (lo > total ? total : lo);
        hi = hi < lo ? lo : (hi > total ? total : hi);
        return (hi - lo + 255) / 256 * 256;
    };
    // P_grp: the groups before grp shared over the workgroup's threads
    int64_t part = 0;
    for (int h = t; h < grp; h += 256) part += kpad(h);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) wsum[wave] = part;
    __syncthreads();
    const int64_t P = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    int64_t K = kpad(grp);
    const int64_t lim = lda < ldb ? lda : ldb;
    // a group whose padded range runs past the operands' width would lose real
    // contraction columns: its outputs are made NaN instead of a short sum (K = -1)
    if (K > 0 && P + K > lim) K = -1;
    const int64_t row0 = pm * big::BM, col0 = pn * big::BN;
    const float* sa_lane = sa + (int64_t)grp * m + (row0 + t < m ? row0 + t : m - 1);
    const float* sb_lane = sb + (int64_t)grp * n + (col0 + t < n ? col0 + t : n - 1);
    v16f acc[4][4];
    if (K > 0) {
        k128_mainloop<FA, FB, false>(smem, a + row0 * lda + P, lda, m - row0, b + col0 * ldb + P, ldb, n - col0, K,
                                     sa_lane, sb_lane, nullptr, nullptr, 0, 0, acc);
    } else {                                             // empty group: 0 * sa * sb (cut: 0 * NaN)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
        float* s_rows = reinterpret_cast<float*>(smem + big::kScaleOff);
        s_rows[t] = K < 0 ? __builtin_nanf("") : *sa_lane;
        s_rows[256 + t] = *sb_lane;
    }
    uint8_t* dg = reinterpret_cast<uint8_t*>(d) + (int64_t)grp * d_group_stride * (OUT_F32 ? 4 : 2);
    big_epilogue<OUT_F32>(smem, acc, dg, ldd, row0, m - row0, col0, n - col0, vec_out);
}

// Persistent dense kernel: at most one workgroup per CU; workgroup w computes
// the tiles w, w + G, w + 2G, .. (G = gridDim.x, a multiple of 8 whenever a
// workgroup has more than one tile, so each keeps its XCD in the XCD-aware
// order). During a tile's last two K steps the stages are loaded with the next
// tile's first two steps; the epilogue then stages its bf16 block through an
// LDS area of its own (16 rows x 128 columns per wavefront at a time), so those
// loads land while it runs and the next tile starts without a load's latency.
// Every tile loads 256 whole rows of each operand: a tile at the bottom or
// right edge is shifted back to end at row m (column n) and stores only the
// rows and columns past the previous tile (with 16-byte stores only where its
// first column keeps them aligned); with m (n) < 256 there is one tile row
// (column) and its loads are clamped. The per-lane load offsets are then the
// same for every tile.
namespace persist {
constexpr int kChunk = 4 * 1024;                     // one wavefront's 16 staged rows
constexpr int kEpiOff = big::kSmem;                  // after the stages and the scale area
constexpr int kSmem = big::kSmem + 4 * kChunk;       // 146 KB
}  // namespace persist

// Epilogue of the tile whose loaded rows start at row0 and columns at col0:
// stores rows row0 + [row_lo, row_hi) and columns col0 + [col_lo, col_hi),
// d = acc * sa_row * sb_col with the tile's 256 row and 256 column scales in
// the scale area; the stages are untouched.
template <bool OUT_F32, bool UNI = false, int EPI = persist::kEpiOff, bool ONE = false>
__device__ __forceinline__ void chunk_epilogue(uint8_t* smem, v16f (&acc)[4][4], void* __restrict__ d, int64_t ldd,
                                               int64_t row0, int row_lo, int row_hi, int64_t col0, int col_lo,
                                               int col_hi, int vec_out) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t wrow0 = row0 + wm * 128, wcol0 = col0 + wn * 128;
    const int rlo = row_lo - wm * 128, rhi = row_hi - wm * 128;      // this wavefront's rows [rlo, rhi)
    const int clo = col_lo - wn * 128, chi = col_hi - wn * 128;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) asm volatile("" : "+a"(acc[mi][ni]));
    const float* s_rows = reinterpret_cast<const float*>(smem + big::kScaleOff);
    const float* s_cols = s_rows + 256;
    float sbj[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) sbj[ni] = s_cols[wn * 128 + ni * 32 + (lane & 31)];
    // UNI: one scale pair for the whole product (both scales scalar), applied
    // as one factor sa * sb
    const float sab = s_rows[0] * s_cols[0];
    if (OUT_F32) {
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (lr < rlo || lr >= rhi) continue;
                const float sai = s_rows[wm * 128 + lr];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int lc = ni * 32 + (lane & 31);
                    if (lc < clo || lc >= chi) continue;
                    reinterpret_cast<float*>(d)[(wrow0 + lr) * ldd + wcol0 + lc] =
                        UNI ? acc[mi][ni][r] * sab : acc[mi][ni][r] * sai * sbj[ni];
                }
            }
        return;
    }
    uint8_t* ep = smem + EPI + wave * persist::kChunk;
    const int cc = lane & 15;
    const bool full_cols = vec_out && 8 * cc >= clo && 8 * cc + 8 <= chi;
    // the wavefront stores all its 128 x 128 outputs as 16-byte vectors
    // (uniform: most tiles), with no per-row or per-column test
    const bool whole = vec_out && rlo <= 0 && rhi >= 128 && clo <= 0 && chi >= 128;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // row groups 8 mi + 4 h .. + 3 (16 rows): groups 2 qq + lane / 32 of the chunk
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                const int q = 2 * h + qq;
                const int g = 8 * mi + 2 * q + (lane >> 5);
                const u32x4 s4 = *reinterpret_cast<const u32x4*>(&s_rows[wm * 128 + 4 * g]);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int r = 4 * q;
                    v2f v01, v23;
                    if constexpr (ONE) {                 // the scales are 1 (MX: applied in the MFMAs)
                        v01 = v2f{acc[mi][ni][r], acc[mi][ni][r + 1]};
                        v23 = v2f{acc[mi][ni][r + 2], acc[mi][ni][r + 3]};
                    } else if constexpr (UNI) {
                        v01 = v2f{acc[mi][ni][r] * sab, acc[mi][ni][r + 1] * sab};
                        v23 = v2f{acc[mi][ni][r + 2] * sab, acc[mi][ni][r + 3] * sab};
                    } else {
                        v01 = v2f{acc[mi][ni][r] * __uint_as_float(s4[0]) * sbj[ni],
                                  acc[mi][ni][r + 1] * __uint_as_float(s4[1]) * sbj[ni]};
                        v23 = v2f{acc[mi][ni][r + 2] * __uint_as_float(s4[2]) * sbj[ni],
                                  acc[mi][ni][r + 3] * __uint_as_float(s4[3]) * sbj[ni]};
                    }
                    uint2 w;
                    w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, v2bf));
                    w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, v2bf));
                    *reinterpret_cast<uint2*>(ep + epi_off(2 * qq + (lane >> 5), 32 * ni + (lane & 31))) = w;
                }
            }
            wait_vmcnt<63, 0>();                         // this wavefront's chunk writes are done
            __builtin_amdgcn_wave_barrier();
            const int gl = lane >> 4;
            const int g = 8 * mi + 4 * h + gl;
            u32x4 un[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) un[k] = *reinterpret_cast<const u32x4*>(ep + epi_off(gl, 8 * cc + 2 * k));
            u32x4 rows[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
                const int wlo = (r >> 1), whi = 2 + (r >> 1);
#pragma unroll
                for (int k = 0; k < 4; ++k) rows[r][k] = __builtin_amdgcn_perm(un[k][whi], un[k][wlo], sel);
            }
            uint16_t* dst0 = reinterpret_cast<uint16_t*>(d) + (wrow0 + 4 * g) * ldd + wcol0 + 8 * cc;
            if (whole) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_nontemporal_store(rows[r], reinterpret_cast<u32x4*>(dst0 + r * ldd));
                continue;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int lr = 4 * g + r;
                if (lr < rlo || lr >= rhi) continue;
                const u32x4 row = rows[r];
                uint16_t* dst = dst0 + r * ldd;
                if (full_cols) {
                    __builtin_nontemporal_store(row, reinterpret_cast<u32x4*>(dst));
                } else {
                    for (int e = 0; e < 8; ++e)
                        if (8 * cc + e >= clo && 8 * cc + e < chi) dst[e] = (uint16_t)(row[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
}

// big_tile_coords in 32-bit arithmetic (tile counts below 2^31), its divisors
// made opaque at each call so that the divisions' setup is not kept live
// across the K loop.
__device__ __forceinline__ void tile_coords32(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n, int64_t* pm,
                                              int64_t* pn) {
    asm volatile("" : "+s"(tiles_m), "+s"(tiles_n));
    const uint32_t nt = tiles_m * tiles_n;
    const uint32_t q = nt / 8, rem = nt % 8;
    const uint32_t xcd = bid % 8, idx = bid / 8;
    const uint32_t t = xcd * q + (xcd < rem ? xcd : rem) + idx;
    constexpr uint32_t gm = 4;
    const uint32_t span = gm * tiles_n;
    const uint32_t first_m = t / span * gm;
    const uint32_t gsize = tiles_m - first_m < gm ? tiles_m - first_m : gm;
    const uint32_t u = t % span;
    *pm = first_m + u % gsize;
    *pn = u / gsize;
}

// A 256 x 128 half tile of the persistent order (defined with the half-tile
// step below).
template <int FA, int FB, bool UNI>
__device__ __forceinline__ void half_tile(uint8_t* smem, const uint8_t* __restrict__ a, int64_t lda,
                                          const uint8_t* __restrict__ b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                          const float* __restrict__ sa, int sa_vec, const float* __restrict__ sb,
                                          int sb_vec, void* __restrict__ d, int64_t ldd, int vec_out, int64_t first,
                                          int64_t hid);

// UNI: both scales scalar (one scale pair for the whole product), applied as
// the single factor sa * sb. After its tile_limit whole tiles (the same number
// for every workgroup) workgroup w < tail_halves takes half w of the remaining
// tiles (a last round of at most half the workgroups runs as twice as many
// 256 x 128 halves, so 2 rem CUs instead of rem finish it).
template <int FA, int FB, bool OUT_F32, bool UNI>
__global__ __launch_bounds__(256, 1) void k_gemm_persist(const uint8_t* __restrict__ a, int64_t lda,
                                                         const uint8_t* __restrict__ b, int64_t ldb, int64_t m,
                                                         int64_t n, int64_t k, const float* __restrict__ sa,
                                                         int sa_vec, const float* __restrict__ sb, int sb_vec,
                                                         void* __restrict__ d, int64_t ldd, int vec_out,
                                                         int64_t tile_limit, int64_t tail_halves) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[persist::kSmem];
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    // tiles 0 .. tile_limit-1 of the order whole (the rest, if any, as halves at the end)
    const int64_t nt = tile_limit, G = gridDim.x;
    const int t = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nk = k / k128::BK;                     // even, >= 2
    // tile (pm, pn): rows loaded from lrow(pm), columns from lcol(pn)
    auto lrow = [&](int64_t pm) {
        const int64_t r = pm * big::BM;
        return (r + big::BM > m && m >= big::BM) ? m - big::BM : r;
    };
    auto lcol = [&](int64_t pn) {
        const int64_t c = pn * big::BN;
        return (c + big::BN > n && n >= big::BN) ? n - big::BN : c;
    };
    uint32_t aoff[8], boff[8];
    k128_lane_offsets(aoff, lda, m);
    k128_lane_offsets(boff, ldb, n);
    int64_t id = blockIdx.x;                             // < nt (grid <= nt)
    int64_t pm, pn;
    tile_coords32((uint32_t)id, (uint32_t)tiles_m, (uint32_t)tiles_n, &pm, &pn);
    int64_t row0 = lrow(pm), col0 = lcol(pn);
    int row_lo = (int)(pm * big::BM - row0), col_lo = (int)(pn * big::BN - col0);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kScaleOff)) + wave * 256;
    auto issue_scales = [&](int64_t r0, int64_t c0) {
        lds_dma4(sbase, sa + (sa_vec ? (r0 + t < m ? r0 + t : m - 1) : 0));
        lds_dma4(sbase + 1024, sb + (sb_vec ? (c0 + t < n ? c0 + t : n - 1) : 0));
    };
    const uint8_t* at = a + row0 * lda;
    const uint8_t* bt = b + col0 * ldb;
    issue_scales(row0, col0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * k128::kStage)) + wave * 8192;
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + i * 1024, at + s * k128::BK, aoff[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + k128::kOpBytes + i * 1024, bt + s * k128::BK, boff[i]);
    }
    wait_vmcnt<16>();                                    // the scales and step 0 landed
    v16f acc[4][4];
    v8i f0[8];
    u32x4 sx[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    __syncthreads();                                     // step 0 (all threads' loads) is in LDS
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        const int j = k128_frag(f);
        f0[j] = big_join(k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 0),
                         k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 1));
    }
    for (;;) {
        const int64_t nid = id + G;
        const int64_t crow0 = row0, ccol0 = col0;
        const int crow_lo = row_lo, ccol_lo = col_lo;
        const uint8_t* nat = at;                         // with no next tile: this tile's own first
        const uint8_t* nbt = bt;                         // steps (valid addresses, never used)
        if (nid < nt) {
            tile_coords32((uint32_t)nid, (uint32_t)tiles_m, (uint32_t)tiles_n, &pm, &pn);
            row0 = lrow(pm);
            col0 = lcol(pn);
            row_lo = (int)(pm * big::BM - row0);
            col_lo = (int)(pn * big::BN - col0);
            nat = a + row0 * lda;
            nbt = b + col0 * ldb;
        }
        // steps p, p+1 load steps p+2, p+3; the last pair loads the next tile's
        // steps 0 and 1, and its second step reads the next tile's first fragments
        // the first step's MFMAs start the sums from zero (no zeroing pass)
        {
            const bool last = 2 >= nk;
            const uint8_t* la = last ? nat : at;
            const uint8_t* lb = last ? nbt : bt;
            const int64_t kl = last ? 0 : 2 * k128::BK;
            k128_step<FA, FB, 0, true, true, false, true, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl, nullptr,
                                                                nullptr, 0, 0);
            k128_step<FA, FB, 1, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl + k128::BK, nullptr,
                                                          nullptr, 0, 0);
        }
        for (int64_t p = 2; p < nk; p += 2) {
            const bool last = p + 2 >= nk;
            const uint8_t* la = last ? nat : at;
            const uint8_t* lb = last ? nbt : bt;
            const int64_t kl = last ? 0 : (p + 2) * k128::BK;
            k128_step<FA, FB, 0, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl, nullptr, nullptr, 0,
                                                          0);
            k128_step<FA, FB, 1, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl + k128::BK, nullptr,
                                                    nullptr, 0, 0);
        }
        at = nat;
        bt = nbt;
        const int64_t rhi = m - crow0, chi = n - ccol0;
        chunk_epilogue<OUT_F32, UNI>(smem, acc, d, ldd, crow0, crow_lo, (int)(rhi < 256 ? rhi : 256), ccol0, ccol_lo,
                                     (int)(chi < 256 ? chi : 256), vec_out && ccol0 % 8 == 0);
        if (nid >= nt) break;
        id = nid;
        __syncthreads();                                 // every wavefront is done with the scale area
        issue_scales(row0, col0);                        // (landed by the next tile's first mid-step wait)
    }
    wait_vmcnt<0>();
    // the tail: tiles tile_limit .. as 256 x 128 halves, one per workgroup
    // (every workgroup has walked the same number of whole tiles)
    if constexpr (!OUT_F32) {
        if ((int64_t)blockIdx.x < tail_halves) {
            __syncthreads();                             // the stages and the scale area are free
            half_tile<FA, FB, UNI>(smem, a, lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, vec_out,
                                   tile_limit, blockIdx.x);
        }
    }
}

// Persistent MX product (bf16 output, k >= 256, more tiles than CUs): the
// tiles of k_gemm_mx taken as k_gemm_persist takes dense ones (the next tile's
// first two K steps, with their scale records, load during the current tile's
// last two; edge tiles shifted back). The block scales are applied inside the
// MFMAs, so the epilogue stores the sums as they are (ONE). LDS: the stages,
// the (unit) scale area and the two record stages of k_gemm_mx, then the chunk
// epilogue's area.
namespace persist_mx {
constexpr int kEpiOff = big::kSmemMx;
constexpr int kSmem = big::kSmemMx + 4 * persist::kChunk;   // 150 KB
}  // namespace persist_mx

template <int FA, int FB>
__global__ __launch_bounds__(256, 1) void k_gemm_persist_mx(const uint8_t* __restrict__ a, int64_t lda,
                                                            const uint8_t* __restrict__ xa, int64_t ld_xa,
                                                            const uint8_t* __restrict__ b, int64_t ldb,
                                                            const uint8_t* __restrict__ xb, int64_t ld_xb, int64_t m,
                                                            int64_t n, int64_t k, void* __restrict__ d, int64_t ldd,
                                                            int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[persist_mx::kSmem];
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    const int64_t nt = tiles_m * tiles_n, G = gridDim.x;
    const int t = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nk = k / k128::BK;                     // even, >= 2
    auto lrow = [&](int64_t pm) {
        const int64_t r = pm * big::BM;
        return (r + big::BM > m && m >= big::BM) ? m - big::BM : r;
    };
    auto lcol = [&](int64_t pn) {
        const int64_t c = pn * big::BN;
        return (c + big::BN > n && n >= big::BN) ? n - big::BN : c;
    };
    // thread t's K-step-0 scale records: A row / B row mx_row(t) of the tile
    const int rt = mx_row(t);
    auto xa_of = [&](int64_t r0) { return xa + 4 * (r0 + rt < m ? r0 + rt : m - 1); };
    auto xb_of = [&](int64_t c0) { return xb + 4 * (c0 + rt < n ? c0 + rt : n - 1); };
    const int64_t xsa = 4 * ld_xa, xsb = 4 * ld_xb;
    uint32_t aoff[8], boff[8];
    k128_lane_offsets(aoff, lda, m);
    k128_lane_offsets(boff, ldb, n);
    int64_t id = blockIdx.x;                             // < nt (grid <= nt)
    int64_t pm, pn;
    tile_coords32((uint32_t)id, (uint32_t)tiles_m, (uint32_t)tiles_n, &pm, &pn);
    int64_t row0 = lrow(pm), col0 = lcol(pn);
    int row_lo = (int)(pm * big::BM - row0), col_lo = (int)(pn * big::BN - col0);
    {
        float* sc = reinterpret_cast<float*>(smem + big::kScaleOff);
        sc[t] = 1.0f;                                    // (ordered by the barrier below)
        sc[256 + t] = 1.0f;
    }
    const uint8_t* at = a + row0 * lda;
    const uint8_t* bt = b + col0 * ldb;
    const uint8_t* xat = xa_of(row0);
    const uint8_t* xbt = xb_of(col0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * k128::kStage)) + wave * 8192;
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + i * 1024, at + s * k128::BK, aoff[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + k128::kOpBytes + i * 1024, bt + s * k128::BK, boff[i]);
        const uint32_t xbase =
            __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kMxOff + s * big::kMxStage)) + wave * 256;
        lds_dma4(xbase, xat + s * xsa);
        lds_dma4(xbase + 1024, xbt + s * xsb);
    }
    wait_vmcnt<18>();                                    // step 0 and its records landed
    v16f acc[4][4];
    v8i f0[8];
    u32x4 sx[2];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        const int j = k128_frag(f);
        f0[j] = big_join(k128_half<true>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 0),
                         k128_half<true>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 1));
    }
    sx[0] = mx_scales(smem + big::kMxOff, 0);
    sx[1] = mx_scales(smem + big::kMxOff, 1);
    for (;;) {
        const int64_t nid = id + G;
        const int64_t crow0 = row0, ccol0 = col0;
        const int crow_lo = row_lo, ccol_lo = col_lo;
        const uint8_t* nat = at;                         // with no next tile: this tile's own first
        const uint8_t* nbt = bt;                         // steps (valid addresses, never used)
        const uint8_t* nxat = xat;
        const uint8_t* nxbt = xbt;
        if (nid < nt) {
            tile_coords32((uint32_t)nid, (uint32_t)tiles_m, (uint32_t)tiles_n, &pm, &pn);
            row0 = lrow(pm);
            col0 = lcol(pn);
            row_lo = (int)(pm * big::BM - row0);
            col_lo = (int)(pn * big::BN - col0);
            nat = a + row0 * lda;
            nbt = b + col0 * ldb;
            nxat = xa_of(row0);
            nxbt = xb_of(col0);
        }
        // the first step's MFMAs start the sums from zero
        {
            const bool last = 2 >= nk;
            const int64_t kl = last ? 0 : 2 * k128::BK;
            k128_step<FA, FB, 0, true, true, true, true, true>(smem, acc, f0, sx, last ? nat : at, aoff,
                                                               last ? nbt : bt, boff, kl, last ? nxat : xat,
                                                               last ? nxbt : xbt, xsa, xsb);
            k128_step<FA, FB, 1, true, true, true, true>(smem, acc, f0, sx, last ? nat : at, aoff, last ? nbt : bt,
                                                         boff, kl + k128::BK, last ? nxat : xat, last ? nxbt : xbt,
                                                         xsa, xsb);
        }
        for (int64_t p = 2; p < nk; p += 2) {
            const bool last = p + 2 >= nk;
            const int64_t kl = last ? 0 : (p + 2) * k128::BK;
            k128_step<FA, FB, 0, true, true, true, true>(smem, acc, f0, sx, last ? nat : at, aoff, last ? nbt : bt,
                                                         boff, kl, last ? nxat : xat, last ? nxbt : xbt, xsa, xsb);
            k128_step<FA, FB, 1, true, true, true, true>(smem, acc, f0, sx, last ? nat : at, aoff, last ? nbt : bt,
                                                         boff, kl + k128::BK, last ? nxat : xat, last ? nxbt : xbt,
                                                         xsa, xsb);
        }
        at = nat;
        bt = nbt;
        xat = nxat;
        xbt = nxbt;
        const int64_t rhi = m - crow0, chi = n - ccol0;
        chunk_epilogue<false, true, persist_mx::kEpiOff, true>(smem, acc, d, ldd, crow0, crow_lo,
                                                         (int)(rhi < 256 ? rhi : 256), ccol0, ccol_lo,
                                                         (int)(chi < 256 ? chi : 256), vec_out && ccol0 % 8 == 0);
        if (nid >= nt) break;
        id = nid;
    }
    wait_vmcnt<0>();
}

// Persistent ragged-K product (bf16 output, at most ragged::kMaxGroups
// groups): the sums of k_grouped_gemm_ragged_k, with the persistent kernel's
// overlap of one tile's epilogue and the next tile's first loads. Each
// workgroup first builds the group table in LDS: padded K_g (-1 for a group
// cut by the operands' width), its start P_g, and the groups ranked by
// decreasing K_g (ties by index). Slot s = r * per8 + w then stands for tile w
// of the group ranked r, w dealt to the XCDs as in k_grouped_gemm_ragged_k;
// workgroup i takes slots i, i + G, i + 2G, .. (G = gridDim.x, a multiple of
// 8, so a workgroup keeps to its XCD's share of every group). Dealing the
// longest contractions first keeps the workgroups' total work even when the
// group sizes are skewed. Edge tiles are shifted back as in k_gemm_persist.
namespace ragged {
constexpr int kMaxGroups = 256;
}  // namespace ragged

__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Persistent grouped product (bf16 output, at most gpersist::kMaxGroups
// groups, at least 256 rows in all): k_grouped_gemm_big's tiles in its
// logical order (each XCD a contiguous run; within a group, runs of 4 m-tiles
// sweep the n-tiles), taken as k_gemm_persist takes dense tiles: the next
// tile's first two K steps load during the current tile's last two. Each
// workgroup keeps the groups' tile prefix sums in LDS for the whole kernel and
// finds each tile's group by binary search. A tile that would run past the
// last row of the token matrix is shifted back to end there (and one past the
// last column of B to end at column n), so every tile loads 256 whole rows with
// one set of lane offsets; the rows it computes outside its group's m-tile
// (another group's tokens, with this group's weights) are never stored.
namespace gpersist {
constexpr int kMaxGroups = 1024;
constexpr int kPreOff = persist::kSmem;                    // after the persistent kernel's LDS
constexpr int kSmem = kPreOff + (kMaxGroups + 1) * 4;      // (G + 1) int32 prefix sums: 150 KB
constexpr int64_t kMaxK = 4096;                            // longer contractions keep k_grouped_gemm_big
}  // namespace gpersist

// One tile of the persistent grouped loop (every field wave-uniform).
struct GpTile {
    int grp;
    int64_t row0, col0;     // first loaded row / column
    int row_lo, row_hi;     // stored rows, relative to row0
    int col_lo;             // first stored column, relative to col0
};

template <int FA, int FB>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_persist(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ b, int64_t ldb, int64_t b_group_stride,
    const int64_t* __restrict__ offsets, int g, int64_t total_m, int64_t n, int64_t k, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ d, int64_t ldd, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[gpersist::kSmem];
    const uint32_t tiles_n = (uint32_t)((n + big::BN - 1) / big::BN);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    auto bounds = [&](int e, int64_t* lo, int64_t* hi) {
        int64_t s = offsets[e], u = offsets[e + 1];
        s = s < 0 ? 0 : (s > total_m ? total_m : s);
        u = u < s ? s : (u > total_m ? total_m : u);
        *lo = s;
        *hi = u;
    };
    // prefix sums of the groups' tile counts (g <= 1024: up to 4 groups per thread)
    int32_t* pre = reinterpret_cast<int32_t*>(smem + gpersist::kPreOff);
    int32_t* wsum = reinterpret_cast<int32_t*>(smem + big::kScaleOff);
    {
        const int per = (g + 255) / 256;
        const int e0 = t * per, e1 = e0 + per < g ? e0 + per : g;
        int32_t mine = 0;
        for (int e = e0; e < e1; ++e) {
            int64_t lo, hi;
            bounds(e, &lo, &hi);
            mine += (int32_t)(((hi - lo + big::BM - 1) / big::BM) * tiles_n);
        }
        int32_t incl = mine;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int32_t run = incl - mine;
        for (uint32_t w = 0; w < wave; ++w) run += wsum[w];
        for (int e = e0; e < e1; ++e) {
            pre[e] = run;
            int64_t lo, hi;
            bounds(e, &lo, &hi);
            run += (int32_t)(((hi - lo + big::BM - 1) / big::BM) * tiles_n);
        }
        if (t == 255) pre[g] = run;
        __syncthreads();                                 // (also: wsum, in the scale area, is dead)
    }
    const uint32_t nt = (uint32_t)__builtin_amdgcn_readfirstlane(pre[g]);
    const uint32_t G = gridDim.x;
    if (blockIdx.x >= nt) return;                        // uniform over the workgroup
    // logical tile of slot id (XCD-aware as k_grouped_gemm_big), its group and place
    auto resolve = [&](uint32_t id, GpTile& tl) {
        uint32_t ntt = nt, tn = tiles_n;
        asm volatile("" : "+s"(ntt), "+s"(tn));
        const uint32_t q = ntt / 8, rem = ntt % 8;
        const uint32_t xcd = id % 8, idx = id / 8;
        uint32_t lt = xcd * q + (xcd < rem ? xcd : rem) + idx;
        int lo_e = 0, hi_e = g;                          // pre[lo_e] <= lt < pre[hi_e]
        while (hi_e - lo_e > 1) {
            const int mid = (lo_e + hi_e) >> 1;
            if ((uint32_t)pre[mid] <= lt)
                lo_e = mid;
            else
                hi_e = mid;
        }
        const int grp = __builtin_amdgcn_readfirstlane(lo_e);
        lt -= (uint32_t)__builtin_amdgcn_readfirstlane(pre[grp]);
        int64_t lo, hi;
        bounds(grp, &lo, &hi);
        lo = uniform64(lo);
        hi = uniform64(hi);
        const uint32_t tm = (uint32_t)((hi - lo + big::BM - 1) / big::BM);
        constexpr uint32_t gm = 4;
        const uint32_t span = gm * tn;
        const uint32_t first_m = lt / span * gm;
        const uint32_t gsize = tm - first_m < gm ? tm - first_m : gm;
        const uint32_t u = lt % span;
        const int64_t pm = first_m + u % gsize, pn = u / gsize;
        const int64_t r = lo + pm * big::BM, c = pn * big::BN;
        tl.grp = grp;
        tl.row0 = r + big::BM > total_m ? total_m - big::BM : r;
        tl.col0 = (c + big::BN > n && n >= big::BN) ? n - big::BN : c;
        tl.row_lo = (int)(r - tl.row0);
        tl.row_hi = (int)((hi < r + big::BM ? hi : r + big::BM) - tl.row0);
        tl.col_lo = (int)(c - tl.col0);
    };
    uint32_t aoff[8], boff[8];
    k128_lane_offsets(aoff, lda, total_m);
    k128_lane_offsets(boff, ldb, n);
    uint32_t id = blockIdx.x;
    GpTile cur;
    resolve(id, cur);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kScaleOff)) + wave * 256;
    auto issue_scales = [&](const GpTile& tl) {
        const int64_t r = tl.row0 + t, c = tl.col0 + t;
        lds_dma4(sbase, sa + (r < total_m ? r : total_m - 1));
        lds_dma4(sbase + 1024, sb + (int64_t)tl.grp * n + (c < n ? c : n - 1));
    };
    const int64_t nk = k / k128::BK;                     // even, >= 2
    const uint8_t* at = a + cur.row0 * lda;
    const uint8_t* bt = b + (int64_t)cur.grp * b_group_stride + cur.col0 * ldb;
    issue_scales(cur);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * k128::kStage)) + wave * 8192;
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + i * 1024, at + s * k128::BK, aoff[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + k128::kOpBytes + i * 1024, bt + s * k128::BK, boff[i]);
    }
    wait_vmcnt<16>();                                    // the scales and step 0 landed
    v16f acc[4][4];
    v8i f0[8];
    u32x4 sx[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    __syncthreads();                                     // step 0 (all threads' loads) is in LDS
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        const int j = k128_frag(f);
        f0[j] = big_join(k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 0),
                         k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 1));
    }
    for (;;) {
        const uint32_t nid = id + G;
        const GpTile done = cur;
        const uint8_t* nat = at;                         // with no next tile: this tile's own first
        const uint8_t* nbt = bt;                         // steps (valid addresses, never used)
        if (nid < nt) {
            resolve(nid, cur);
            nat = a + cur.row0 * lda;
            nbt = b + (int64_t)cur.grp * b_group_stride + cur.col0 * ldb;
        }
        // the first step's MFMAs start the sums from zero (no zeroing pass)
        for (int64_t p = 0; p < nk; p += 2) {            // nk >= 2
            const bool last = p + 2 >= nk;
            const uint8_t* la = last ? nat : at;
            const uint8_t* lb = last ? nbt : bt;
            const int64_t kl = last ? 0 : (p + 2) * k128::BK;
            if (p == 0)
                k128_step<FA, FB, 0, true, true, false, true, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl, nullptr,
                                                                    nullptr, 0, 0);
            else
                k128_step<FA, FB, 0, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl, nullptr,
                                                              nullptr, 0, 0);
            k128_step<FA, FB, 1, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl + k128::BK, nullptr,
                                                          nullptr, 0, 0);
        }
        at = nat;
        bt = nbt;
        const int64_t chi = n - done.col0;
        chunk_epilogue<false>(smem, acc, d, ldd, done.row0, done.row_lo, done.row_hi, done.col0, done.col_lo,
                              (int)(chi < 256 ? chi : 256), vec_out && done.col0 % 8 == 0);
        if (nid >= nt) break;
        id = nid;
        __syncthreads();                                 // every wavefront is done with the scale area
        issue_scales(cur);                               // (landed by the next tile's first mid-step wait)
    }
    wait_vmcnt<0>();
}

// One tile of the persistent ragged-K loop (every field wave-uniform).
struct RaggedTile {
    uint32_t slot;
    int grp;
    int32_t k;              // padded contraction length; 0: empty group, -1: cut
    int64_t p;              // first contraction column
    int64_t row0, col0;     // first loaded row / column
    int row_lo, col_lo;     // first stored row / column, relative to row0 / col0
};

template <int FA, int FB>
__global__ __launch_bounds__(256, 1) void k_grouped_gemm_ragged_k_persist(
    const uint8_t* __restrict__ a, int64_t lda, const uint8_t* __restrict__ b, int64_t ldb,
    const int64_t* __restrict__ offsets, int G, int64_t total, int64_t m, int64_t n, const float* __restrict__ sa,
    const float* __restrict__ sb, void* __restrict__ d, int64_t ldd, int64_t d_group_stride, int vec_out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[persist::kSmem];
    __shared__ int64_t g_start[ragged::kMaxGroups];
    __shared__ int32_t g_k[ragged::kMaxGroups];
    __shared__ int32_t g_by_rank[ragged::kMaxGroups];
    const int t = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // group table (G <= 256 = the thread count)
    int32_t kp = 0;
    if (t < G) {
        int64_t lo = offsets[t], hi = offsets[t + 1];
        lo = lo < 0 ? 0 : (lo > total ? total : lo);
        hi = hi < lo ? lo : (hi > total ? total : hi);
        kp = (int32_t)((hi - lo + 255) / 256 * 256);
    }
    g_k[t] = kp;
    __syncthreads();
    int64_t pstart = 0;
    for (int h = 0; h < t && h < G; ++h) pstart += g_k[h];
    const int64_t lim = lda < ldb ? lda : ldb;
    __syncthreads();                                     // every thread has read g_k
    if (t < G) {
        g_start[t] = pstart;
        // a padded range past the operands' width would lose contraction columns
        if (kp > 0 && pstart + kp > lim) g_k[t] = -1;
    }
    __syncthreads();
    if (t < G) {
        const int32_t kt = g_k[t];
        int r = 0;
        for (int h = 0; h < G; ++h) {
            const int32_t kh = g_k[h];
            r += (kh > kt) || (kh == kt && h < t);
        }
        g_by_rank[r] = t;
    }
    __syncthreads();

    const uint32_t tiles_m = (uint32_t)((m + big::BM - 1) / big::BM), tiles_n = (uint32_t)((n + big::BN - 1) / big::BN);
    const uint32_t per = tiles_m * tiles_n, per8 = (per + 7) / 8 * 8;
    const uint32_t slots = (uint32_t)G * per8, gd = gridDim.x;
    auto resolve = [&](uint32_t s, RaggedTile& tl) -> bool {
        uint32_t tm = tiles_m, tn = tiles_n, p8 = per8;
        asm volatile("" : "+s"(tm), "+s"(tn), "+s"(p8));
        const uint32_t q = tm * tn / 8, rem = tm * tn % 8;
        for (; s < slots; s += gd) {
            const uint32_t r = s / p8, w = s % p8;
            const uint32_t xcd = w % 8, idx = w / 8;
            if (idx >= q + (xcd < rem ? 1u : 0u)) continue;
            const uint32_t lt = xcd * q + (xcd < rem ? xcd : rem) + idx;
            constexpr uint32_t gm = 4;
            const uint32_t span = gm * tn;
            const uint32_t first_m = lt / span * gm;
            const uint32_t gsize = tm - first_m < gm ? tm - first_m : gm;
            const uint32_t u = lt % span;
            const int64_t pm = first_m + u % gsize, pn = u / gsize;
            tl.slot = s;
            tl.grp = __builtin_amdgcn_readfirstlane(g_by_rank[r]);
            tl.k = __builtin_amdgcn_readfirstlane(g_k[tl.grp]);
            tl.p = uniform64(g_start[tl.grp]);
            const int64_t r0 = pm * big::BM, c0 = pn * big::BN;
            tl.row0 = (r0 + big::BM > m && m >= big::BM) ? m - big::BM : r0;
            tl.col0 = (c0 + big::BN > n && n >= big::BN) ? n - big::BN : c0;
            tl.row_lo = (int)(r0 - tl.row0);
            tl.col_lo = (int)(c0 - tl.col0);
            return true;
        }
        return false;
    };
    RaggedTile cur;
    if (!resolve(blockIdx.x, cur)) return;               // uniform over the workgroup
    uint32_t aoff[8], boff[8];
    k128_lane_offsets(aoff, lda, m);
    k128_lane_offsets(boff, ldb, n);
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(smem + big::kScaleOff)) + wave * 256;
    auto issue_scales = [&](const RaggedTile& tl) {
        const int64_t r = tl.row0 + t, c = tl.col0 + t;
        lds_dma4(sbase, sa + (int64_t)tl.grp * m + (r < m ? r : m - 1));
        lds_dma4(sbase + 1024, sb + (int64_t)tl.grp * n + (c < n ? c : n - 1));
    };
    issue_scales(cur);
    bool loaded = false;                                 // the stages hold cur's steps 0 and 1
    v16f acc[4][4];
    v8i f0[8];
    u32x4 sx[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    for (;;) {
        RaggedTile nxt;
        const bool more = resolve(cur.slot + gd, nxt);
        const uint8_t* at = a + cur.row0 * lda + cur.p;
        const uint8_t* bt = b + cur.col0 * ldb + cur.p;
        if (cur.k > 0 && !loaded) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * k128::kStage)) + wave * 8192;
#pragma unroll
                for (int i = 0; i < 8; ++i) lds_dma16_s(base + i * 1024, at + s * k128::BK, aoff[i]);
#pragma unroll
                for (int i = 0; i < 8; ++i) lds_dma16_s(base + k128::kOpBytes + i * 1024, bt + s * k128::BK, boff[i]);
            }
            wait_vmcnt<16>();                            // everything before step 1's loads landed
            __syncthreads();
#pragma unroll
            for (int f = 0; f < 8; ++f) {
                const int j = k128_frag(f);
                f0[j] = big_join(k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 0),
                                 k128_half<false>(j < 4 ? smem : smem + k128::kOpBytes, big_row(j), 0, 1));
            }
        }
        const int64_t rhi = m - cur.row0, chi = n - cur.col0;
        uint8_t* dg = reinterpret_cast<uint8_t*>(d) + (int64_t)cur.grp * d_group_stride * 2;
        const int row_hi = (int)(rhi < 256 ? rhi : 256), col_hi = (int)(chi < 256 ? chi : 256);
        const int vo = vec_out && cur.col0 % 8 == 0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
        if (cur.k > 0) {
            // steps p, p+1 load steps p+2, p+3; the last pair loads the next
            // tile's steps 0 and 1 when it has a contraction (else this tile's
            // own first steps again: valid addresses, never used)
            const bool pre = more && nxt.k > 0;
            const uint8_t* nat = pre ? a + nxt.row0 * lda + nxt.p : at;
            const uint8_t* nbt = pre ? b + nxt.col0 * ldb + nxt.p : bt;
            const int64_t nk = cur.k / k128::BK;         // even, >= 2
            int64_t p = 0;
            do {
                const bool last = p + 2 >= nk;
                const uint8_t* la = last ? nat : at;
                const uint8_t* lb = last ? nbt : bt;
                const int64_t kl = last ? 0 : (p + 2) * k128::BK;
                k128_step<FA, FB, 0, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl, nullptr,
                                                              nullptr, 0, 0);
                k128_step<FA, FB, 1, true, true, false, true>(smem, acc, f0, sx, la, aoff, lb, boff, kl + k128::BK,
                                                              nullptr, nullptr, 0, 0);
                p += 2;
            } while (p < nk);
            loaded = pre;
            chunk_epilogue<false>(smem, acc, dg, ldd, cur.row0, cur.row_lo, row_hi, cur.col0, cur.col_lo, col_hi, vo);
        } else {                                         // empty group: 0 * sa * sb (cut: NaN row scales)
            wait_vmcnt<0>();
            __syncthreads();                             // every thread's scale loads landed
            if (cur.k < 0) {
                reinterpret_cast<float*>(smem + big::kScaleOff)[t] = __builtin_nanf("");
                __syncthreads();
            }
            loaded = false;
            // (its own epilogue call: the sums of the K loop and these zeros
            // keep separate registers, with no copies between them)
            v16f zero[4][4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
#pragma unroll
                    for (int r = 0; r < 16; ++r) zero[mi][ni][r] = 0.0f;
            chunk_epilogue<false>(smem, zero, dg, ldd, cur.row0, cur.row_lo, row_hi, cur.col0, cur.col_lo, col_hi,
                                  vo);
        }
        if (!more) break;
        cur = nxt;
        __syncthreads();                                 // every wavefront is done with the scale area
        issue_scales(cur);                               // (landed by the next mid-step wait, or waited for above)
    }
    wait_vmcnt<0>();
}

// Half tiles (256 x 128) for the last, partial round of the persistent dense
// product: when the tiles left after the full rounds are at most half a round,
// they run as twice as many 256 x 128 halves at the end of the persistent
// kernel (half_tile) instead of leaving most CUs idle while a few finish them. Four wavefronts, each owning
// 128 x 64 outputs (4 x 2 blocks of 32 x 32); the K128 step of the large-tile
// kernels with 8 MFMAs per K half per wavefront and B's 128 rows in a 16 KB
// operand; each wavefront stages its results through LDS one 32-row chunk at a
// time.
namespace t128 {
constexpr int BM = 256, BN = 128;
constexpr int kAOp = BM * 128;                    // A of a K128 stage: 32 KB
constexpr int kStage = kAOp + BN * 128;           // 48 KB
constexpr int kScaleOff = 2 * kStage;             // 256 row + 128 column scales
constexpr int kChunkOff = kScaleOff + (BM + BN) * 4;
constexpr int kChunk = 32 * 64 * 2;               // a wavefront's staged 32 x 64 bf16 chunk
constexpr int kSmem = kChunkOff + 4 * kChunk;     // 113.5 KB
}  // namespace t128
static_assert(t128::kSmem <= persist::kSmem, "the half tiles run in the persistent kernel's LDS");

// Fragment rows of the 256 x 128 tile: j < 4: A block j of the wavefront's
// 128 rows; j = 4, 5: B block j - 4 of its 64 columns (rows of B).
__device__ __forceinline__ int t128_row(int j) {
    const int w = threadIdx.x >> 6;
    return (j < 4 ? (w >> 1) * 128 + j * 32 : (w & 1) * 64 + (j - 4) * 32) + (threadIdx.x & 31);
}
// Fragment order of a step: A0, B0, B1, A1, A2, A3 (the MFMA sweep (mi, ni) =
// (0,0), (0,1), (1,0), .. first needs them in that order).
__device__ __forceinline__ int t128_frag(int f) { return f == 0 ? 0 : (f <= 2 ? f + 3 : f - 2); }

// B's 4 loads per thread of a step (128 rows): load i of wavefront w fills rows
// w * 32 + 8i .. + 7, as k128_lane_offsets does for A's 256 rows.
__device__ __forceinline__ void t128_lane_offsets_b(uint32_t (&off)[4], int64_t ld, int64_t valid_rows) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t ld32 = (uint32_t)ld;
    const int last = (int)(valid_rows < 128 ? valid_rows : 128) - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = wave * 32 + i * 8 + (lane >> 3);
        const int chunk = k128_slot(row, lane & 7);
        const uint32_t r = (uint32_t)(row < last ? row : last);
        off[i] = r * ld32 + (uint32_t)(chunk * 16);
    }
}

// One K128 step of the 256 x 128 tile (the k128_step scheme: 8 MFMAs per K
// half per wavefront, the second half's fragments read during the first half,
// a mid-step wait and barrier, then the next step's first-half fragments read
// and step p+2's 12 loads per thread issued during the second half).
template <int FA, int FB, int CUR, bool NEXT, bool LOADS>
__device__ __forceinline__ void t128_step(uint8_t* smem, v16f (&acc)[4][2], v8i (&f0)[6], const uint8_t* a,
                                         const uint32_t (&aoff)[8], const uint8_t* b, const uint32_t (&boff)[4],
                                         int64_t knext, bool issue = true) {
    const uint8_t* ta = smem + CUR * t128::kStage;
    const uint8_t* tb = ta + t128::kAOp;
    const uint8_t* na = smem + (CUR ^ 1) * t128::kStage;
    const uint8_t* nb = na + t128::kAOp;
    u32x4 h1[12];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int mi = i >> 1, ni = i & 1;
        acc[mi][ni] = mfma64<FA, FB, false, 0>(f0[mi], f0[4 + ni], acc[mi][ni], 0u, 0u);
        if (i < 6) {
            const int j = t128_frag(i);
            h1[2 * i] = k128_half<false>(j < 4 ? ta : tb, t128_row(j), 1, 0);
            h1[2 * i + 1] = k128_half<false>(j < 4 ? ta : tb, t128_row(j), 1, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    v8i f1[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) f1[t128_frag(f)] = big_join(h1[2 * f], h1[2 * f + 1]);
    wait_vmcnt<0, 0>();
    __syncthreads();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + CUR * t128::kStage));
    u32x4 h0[12];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int mi = i >> 1, ni = i & 1;
        acc[mi][ni] = mfma64<FA, FB, false, 2>(f1[mi], f1[4 + ni], acc[mi][ni], 0u, 0u);
        if (NEXT && i < 6) {
            const int j = t128_frag(i);
            h0[2 * i] = k128_half<false>(j < 4 ? na : nb, t128_row(j), 0, 0);
            h0[2 * i + 1] = k128_half<false>(j < 4 ? na : nb, t128_row(j), 0, 1);
        }
        if (LOADS && issue) {
            lds_dma16_s(base + wave * 8192 + i * 1024, a + knext, aoff[i]);
            if (i >= 4) lds_dma16_s(base + t128::kAOp + wave * 4096 + (i - 4) * 1024, b + knext, boff[i - 4]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (NEXT) {
#pragma unroll
        for (int f = 0; f < 6; ++f) f0[t128_frag(f)] = big_join(h0[2 * f], h0[2 * f + 1]);
    }
}

// The output block a chunk stores into.
struct T128Out {
    uint8_t* d;
    int64_t row0, col0;     // first loaded row / column
    int row_lo, row_hi;     // stored rows, relative to row0
    int col_lo, col_hi;     // stored columns, relative to col0
    int vec;                // 16-byte stores allowed
};

// Chunk MI of a finished tile: rows wm * 128 + 32 MI .. + 31, the wavefront's
// 64 columns; d = acc * sa_row * sb_col, staged through the wavefront's LDS
// chunk (4-row groups g: column c at g * 512 + unit (c / 2, swizzled) * 16 +
// (c % 2) * 8) and stored as 16-byte row pieces, 8 lanes per 128-byte row.
template <int MI, bool UNI>
__device__ __forceinline__ void t128_chunk(uint8_t* smem, v16f (&acc)[4][2], const T128Out& o, int64_t ldd) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    asm volatile("" : "+a"(acc[MI][0]));
    asm volatile("" : "+a"(acc[MI][1]));
    const float* s_rows = reinterpret_cast<const float*>(smem + t128::kScaleOff);
    const float* s_cols = s_rows + t128::BM;
    const int r0 = wm * 128 + MI * 32;                   // first tile row of the chunk
    const int c0 = wn * 64;                              // first tile column of the wavefront
    uint8_t* ep = smem + t128::kChunkOff + wave * t128::kChunk;
    auto off = [](int g, int c) {
        const int u = c >> 1;
        return g * 512 + (((u & ~3) | ((u ^ (u >> 3)) & 3)) << 4) + ((c & 1) << 3);
    };
    const float sab = s_rows[0] * s_cols[0];             // UNI: one scale pair, one factor
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const float sb = s_cols[c0 + ni * 32 + (lane & 31)];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int g = 2 * q + (lane >> 5);           // rows 4g .. 4g+3 of the chunk
            const u32x4 s4 = *reinterpret_cast<const u32x4*>(&s_rows[r0 + 4 * g]);
            const int r = 4 * q;
            v2f v01, v23;
            if constexpr (UNI) {
                v01 = v2f{acc[MI][ni][r] * sab, acc[MI][ni][r + 1] * sab};
                v23 = v2f{acc[MI][ni][r + 2] * sab, acc[MI][ni][r + 3] * sab};
            } else {
                v01 = v2f{acc[MI][ni][r] * __uint_as_float(s4[0]) * sb, acc[MI][ni][r + 1] * __uint_as_float(s4[1]) * sb};
                v23 = v2f{acc[MI][ni][r + 2] * __uint_as_float(s4[2]) * sb,
                          acc[MI][ni][r + 3] * __uint_as_float(s4[3]) * sb};
            }
            uint2 w;
            w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v01, v2bf));
            w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v23, v2bf));
            *reinterpret_cast<uint2*>(ep + off(g, ni * 32 + (lane & 31))) = w;
        }
    }
    wait_vmcnt<63, 0>();                                 // this wavefront's staging writes are done
    __builtin_amdgcn_wave_barrier();
    const int cc = lane & 7;                             // columns 8cc .. 8cc+7 of the wavefront's 64
    const int g = lane >> 3;                             // rows 4g .. 4g+3 of the chunk
    u32x4 un[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) un[k] = *reinterpret_cast<const u32x4*>(ep + off(g, 8 * cc + 2 * k));
    const bool full = o.vec && r0 >= o.row_lo && r0 + 32 <= o.row_hi && c0 >= o.col_lo && c0 + 64 <= o.col_hi;
    const int clo = o.col_lo - c0, chi = o.col_hi - c0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int lr = r0 + 4 * g + r;                   // tile row
        const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
        const int wlo = (r >> 1), whi = 2 + (r >> 1);
        u32x4 row;
#pragma unroll
        for (int k = 0; k < 4; ++k) row[k] = __builtin_amdgcn_perm(un[k][whi], un[k][wlo], sel);
        uint16_t* dst = reinterpret_cast<uint16_t*>(o.d) + (o.row0 + lr) * ldd + o.col0 + c0 + 8 * cc;
        if (full) {
            __builtin_nontemporal_store(row, reinterpret_cast<u32x4*>(dst));
        } else if (lr >= o.row_lo && lr < o.row_hi) {
            for (int e = 0; e < 8; ++e)
                if (8 * cc + e >= clo && 8 * cc + e < chi) dst[e] = (uint16_t)(row[e >> 1] >> (16 * (e & 1)));
        }
    }
}


// One 256 x 128 half of tile `first + blockIdx.x / 2` in k_gemm_persist's
// order: the tile's rows and columns as that kernel would take them (edge
// tiles shifted back), the half's 128 columns from col0 + 128 (blockIdx.x % 2).
// Half hid of the tile `first + hid / 2` of the persistent order (half
// hid % 2: its first or last 128 columns), with t128::kSmem bytes of LDS at
// smem; every branch is uniform over the workgroup.
template <int FA, int FB, bool UNI>
__device__ __forceinline__ void half_tile(uint8_t* smem, const uint8_t* __restrict__ a, int64_t lda,
                                          const uint8_t* __restrict__ b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                                          const float* __restrict__ sa, int sa_vec, const float* __restrict__ sb,
                                          int sb_vec, void* __restrict__ d, int64_t ldd, int vec_out, int64_t first,
                                          int64_t hid) {
    const int64_t tiles_m = (m + big::BM - 1) / big::BM, tiles_n = (n + big::BN - 1) / big::BN;
    int64_t pm, pn;
    tile_coords32((uint32_t)(first + hid / 2), (uint32_t)tiles_m, (uint32_t)tiles_n, &pm, &pn);
    const int hsel = (int)(hid & 1);
    const int64_t r = pm * big::BM, c = pn * big::BN;
    const int64_t row0 = (r + big::BM > m && m >= big::BM) ? m - big::BM : r;
    const int64_t col0 = (c + big::BN > n && n >= big::BN) ? n - big::BN : c;
    const int64_t hc0 = col0 + 128 * hsel;               // the half's first column
    if (hc0 >= n) return;                                // (n < 256: no second half; uniform)
    T128Out o;
    o.d = reinterpret_cast<uint8_t*>(d);
    o.row0 = row0;
    o.col0 = hc0;
    o.row_lo = (int)(r - row0);
    o.row_hi = (int)(m - row0 < big::BM ? m - row0 : big::BM);
    const int64_t clo = c - hc0, chi = (n - col0 < big::BN ? n - col0 : big::BN) - 128 * hsel;
    o.col_lo = (int)(clo > 0 ? clo : 0);
    o.col_hi = (int)(chi < 128 ? chi : 128);
    o.vec = vec_out && hc0 % 8 == 0;
    if (o.col_hi <= o.col_lo) return;                    // nothing of this half is stored (uniform)
    const int t = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint32_t aoff[8], boff[4];
    k128_lane_offsets(aoff, lda, m);
    t128_lane_offsets_b(boff, ldb, n - hc0);
    const uint8_t* at = a + row0 * lda;
    const uint8_t* bt = b + hc0 * ldb;
    {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + t128::kScaleOff));
        const int64_t rr = row0 + t, cc = hc0 + t;
        lds_dma4(base + wave * 256, sa + (sa_vec ? (rr < m ? rr : m - 1) : 0));
        if (wave < 2) lds_dma4(base + t128::BM * 4 + wave * 256, sb + (sb_vec ? (cc < n ? cc : n - 1) : 0));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(smem + s * t128::kStage));
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16_s(base + wave * 8192 + i * 1024, at + s * k128::BK, aoff[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_dma16_s(base + t128::kAOp + wave * 4096 + i * 1024, bt + s * k128::BK, boff[i]);
    }
    wait_vmcnt<12>();                                    // the scales and step 0 landed
    __syncthreads();
    v8i f0[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int j = t128_frag(f);
        f0[j] = big_join(k128_half<false>(j < 4 ? smem : smem + t128::kAOp, t128_row(j), 0, 0),
                         k128_half<false>(j < 4 ? smem : smem + t128::kAOp, t128_row(j), 0, 1));
    }
    v16f acc[4][2];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[mi][ni][q] = 0.0f;
    const int64_t nk = k / k128::BK;                     // even, >= 2
    int64_t p = 0;
    do {                                                 // one path (the last pair loads nothing)
        const bool more = p + 2 < nk;
        t128_step<FA, FB, 0, true, true>(smem, acc, f0, at, aoff, bt, boff, (p + 2) * k128::BK, more);
        t128_step<FA, FB, 1, true, true>(smem, acc, f0, at, aoff, bt, boff, (p + 3) * k128::BK, more);
        p += 2;
    } while (p < nk);
    t128_chunk<0, UNI>(smem, acc, o, ldd);
    t128_chunk<1, UNI>(smem, acc, o, ldd);
    t128_chunk<2, UNI>(smem, acc, o, ldd);
    t128_chunk<3, UNI>(smem, acc, o, ldd);
}

template <int FA, int FB, bool OUT_F32>
hipError_t gemm_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                      const float* sa, int sa_vec, const float* sb, int sb_vec, void* d, int64_t ldd,
                      hipStream_t st) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    const int64_t big_tiles = ((m + big::BM - 1) / big::BM) * ((n + big::BN - 1) / big::BN);
    if (k > 0 && k % 256 == 0 && big_tiles >= 128 && lda < (1 << 24) && ldb < (1 << 24)) {
        const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0;
        const int64_t cus = current_device_props().cus;
        // more tiles than CUs, bf16 output: the persistent kernel (its fp32
        // epilogue would spill, and with one tile per workgroup it gains nothing)
        if constexpr (!OUT_F32) {
            if (big_tiles > cus && cus >= 8 && big_tiles < ((int64_t)1 << 31)) {
                // a last round of at most half the workgroups runs as twice as many 256 x 128 halves
                const int64_t grid = cus / 8 * 8, rem = big_tiles % grid;
                const int64_t limit = (rem > 0 && 2 * rem <= grid) ? big_tiles - rem : big_tiles;
                // scalar scales take the kernel's one-factor epilogue
                const int64_t halves = limit < big_tiles ? 2 * rem : 0;
                if (!sa_vec && !sb_vec)
                    hipLaunchKernelGGL((k_gemm_persist<FA, FB, false, true>), dim3((unsigned)grid), dim3(256), 0, st, a,
                                       lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, vec_out, limit, halves);
                else
                    hipLaunchKernelGGL((k_gemm_persist<FA, FB, false, false>), dim3((unsigned)grid), dim3(256), 0, st, a,
                                       lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, vec_out, limit, halves);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((k_gemm_big<FA, FB, OUT_F32>), dim3((unsigned)big_tiles), dim3(256), 0, st, a, lda, b, ldb,
                           m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, vec_out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_gemm<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, st, a, lda, b, ldb, m, n,
                       k, sa, sa_vec, sb, sb_vec, d, ldd);
    return hipGetLastError();
}

template <int FA, int FB, bool OUT_F32>
hipError_t grouped_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t stride,
                         const int64_t* offsets, int g, int64_t total_m, int64_t n, int64_t k, const float* sa,
                         const float* sb, void* d, int64_t ldd, hipStream_t st) {
    const int64_t tiles = ((total_m + BM - 1) / BM + g) * ((n + BN - 1) / BN);
    if (total_m == 0 || n == 0) return hipSuccess;
    const int64_t big_est = ((total_m + big::BM - 1) / big::BM) * ((n + big::BN - 1) / big::BN);
    if (k > 0 && k % 256 == 0 && big_est >= 128 && g <= kMaxGroupsBig && lda < (1 << 24) &&
        ldb < (1 << 24)) {
        const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0;
        const int64_t grid = ((total_m + big::BM - 1) / big::BM + g) * ((n + big::BN - 1) / big::BN);
        const int64_t cus = current_device_props().cus;
        // bf16 output, short contractions, more tile slots than CUs: the persistent kernel
        if constexpr (!OUT_F32) {
            if (k <= gpersist::kMaxK && g <= gpersist::kMaxGroups && total_m >= big::BM && cus >= 8 && grid > cus &&
                grid < ((int64_t)1 << 31)) {
                hipLaunchKernelGGL((k_grouped_gemm_persist<FA, FB>), dim3((unsigned)(cus / 8 * 8)), dim3(256), 0, st,
                                   a, lda, b, ldb, stride, offsets, g, total_m, n, k, sa, sb, d, ldd, vec_out);
                return hipGetLastError();
            }
        }
        const uint8_t* none = nullptr;
        hipLaunchKernelGGL((k_grouped_gemm_big<FA, FB, OUT_F32, false>), dim3((unsigned)grid), dim3(256), 0, st, a,
                           lda, b, ldb, stride, offsets, g, total_m, n, k, sa, sb, d, ldd, vec_out, none, (int64_t)0,
                           none, (int64_t)0, (int64_t)0);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_grouped_gemm<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, st, a, lda, b, ldb,
                       stride, offsets, g, total_m, n, k, sa, sb, d, ldd);
    return hipGetLastError();
}

// The MX products always take the large-tile kernels (rows and columns past
// the operands are clamped; k % 256 == 0 and lda, ldb < 2^24 are checked by
// the caller).
template <int FA, int FB, bool OUT_F32>
hipError_t gemm_mx_typed(const uint8_t* a, int64_t lda, const uint8_t* xa, int64_t ld_xa, const uint8_t* b,
                         int64_t ldb, const uint8_t* xb, int64_t ld_xb, int64_t m, int64_t n, int64_t k, void* d,
                         int64_t ldd, hipStream_t st) {
    const int64_t tiles = ((m + big::BM - 1) / big::BM) * ((n + big::BN - 1) / big::BN);
    if (tiles == 0) return hipSuccess;
    const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0;
    if constexpr (!OUT_F32) {
        const int64_t cus = current_device_props().cus;
        if (k > 0 && tiles > cus && cus >= 8 && tiles < ((int64_t)1 << 31)) {
            hipLaunchKernelGGL((k_gemm_persist_mx<FA, FB>), dim3((unsigned)(cus / 8 * 8)), dim3(256), 0, st, a, lda,
                               xa, ld_xa, b, ldb, xb, ld_xb, m, n, k, d, ldd, vec_out);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_gemm_mx<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(256), 0, st, a, lda, xa, ld_xa, b,
                       ldb, xb, ld_xb, m, n, k, d, ldd, vec_out);
    return hipGetLastError();
}

template <int FA, int FB, bool OUT_F32>
hipError_t grouped_mx_typed(const uint8_t* a, int64_t lda, const uint8_t* xa, int64_t ld_xa, const uint8_t* b,
                            int64_t ldb, int64_t stride, const uint8_t* xb, int64_t ld_xb, int64_t xstride,
                            const int64_t* offsets, int g, int64_t total_m, int64_t n, int64_t k, void* d, int64_t ldd,
                            hipStream_t st) {
    if (total_m == 0 || n == 0) return hipSuccess;
    const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0;
    const int64_t grid = ((total_m + big::BM - 1) / big::BM + g) * ((n + big::BN - 1) / big::BN);
    const float* none = nullptr;
    hipLaunchKernelGGL((k_grouped_gemm_big<FA, FB, OUT_F32, true>), dim3((unsigned)grid), dim3(256), 0, st, a, lda, b,
                       ldb, stride, offsets, g, total_m, n, k, none, none, d, ldd, vec_out, xa, ld_xa, xb, ld_xb,
                       xstride);
    return hipGetLastError();
}

template <int FA, int FB, bool OUT_F32>
hipError_t ragged_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, const int64_t* offsets, int g,
                        int64_t total, int64_t m, int64_t n, const float* sa, const float* sb, void* d, int64_t ldd,
                        int64_t dgs, hipStream_t st) {
    if (m == 0 || n == 0) return hipSuccess;
    const int64_t per = ((m + big::BM - 1) / big::BM) * ((n + big::BN - 1) / big::BN);
    const int64_t grid = (int64_t)g * ((per + 7) / 8 * 8);
    const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0 && dgs % 8 == 0;
    const int64_t cus = current_device_props().cus;
    // bf16 output, at most 256 groups, more tiles than CUs: the persistent kernel
    if constexpr (!OUT_F32) {
        const int64_t slots = (int64_t)g * ((per + 7) / 8 * 8);
        if (g <= ragged::kMaxGroups && cus >= 8 && slots > cus && slots < ((int64_t)1 << 31)) {
            hipLaunchKernelGGL((k_grouped_gemm_ragged_k_persist<FA, FB>), dim3((unsigned)(cus / 8 * 8)), dim3(256), 0,
                               st, a, lda, b, ldb, offsets, g, total, m, n, sa, sb, d, ldd, dgs, vec_out);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_grouped_gemm_ragged_k<FA, FB, OUT_F32>), dim3((unsigned)grid), dim3(256), 0, st, a, lda, b,
                       ldb, offsets, g, total, m, n, sa, sb, d, ldd, dgs, vec_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_ragged_k(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                                        const int64_t* offsets, int g, int64_t total_m, int64_t m, int64_t n,
                                        const float* sa, const float* sb, void* d, int out_f32, int64_t ldd,
                                        int64_t d_group_stride, hipStream_t st) {
#define CALL(FA, FB, OF) \
    ragged_typed<FA, FB, OF>(a, lda, b, ldb, offsets, g, total_m, m, n, sa, sb, d, ldd, d_group_stride, st)
#define BY_OUT(FA, FB) return out_f32 ? CALL(FA, FB, true) : CALL(FA, FB, false)
    if (fa == kE4M3 && fb == kE4M3) BY_OUT(kE4M3, kE4M3);
    if (fa == kE4M3 && fb == kE5M2) BY_OUT(kE4M3, kE5M2);
    if (fa == kE5M2 && fb == kE4M3) BY_OUT(kE5M2, kE4M3);
    BY_OUT(kE5M2, kE5M2);
#undef BY_OUT
#undef CALL
}

hipError_t launch_gemm_mx(const uint8_t* a, int fa, int64_t lda, const uint8_t* xa, int64_t ld_xa, const uint8_t* b,
                          int fb, int64_t ldb, const uint8_t* xb, int64_t ld_xb, int64_t m, int64_t n, int64_t k,
                          void* d, int out_f32, int64_t ldd, hipStream_t st) {
#define CALL(FA, FB, OF) gemm_mx_typed<FA, FB, OF>(a, lda, xa, ld_xa, b, ldb, xb, ld_xb, m, n, k, d, ldd, st)
#define BY_OUT(FA, FB) return out_f32 ? CALL(FA, FB, true) : CALL(FA, FB, false)
    if (fa == kE4M3 && fb == kE4M3) BY_OUT(kE4M3, kE4M3);
    if (fa == kE4M3 && fb == kE5M2) BY_OUT(kE4M3, kE5M2);
    if (fa == kE5M2 && fb == kE4M3) BY_OUT(kE5M2, kE4M3);
    BY_OUT(kE5M2, kE5M2);
#undef BY_OUT
#undef CALL
}

hipError_t launch_grouped_gemm_mx(const uint8_t* a, int fa, int64_t lda, const uint8_t* xa, int64_t ld_xa,
                                  const uint8_t* b, int fb, int64_t ldb, int64_t b_group_stride, const uint8_t* xb,
                                  int64_t ld_xb, int64_t xb_group_stride, const int64_t* offsets, int g,
                                  int64_t total_m, int64_t n, int64_t k, void* d, int out_f32, int64_t ldd,
                                  hipStream_t st) {
#define CALL(FA, FB, OF)                                                                                        \
    grouped_mx_typed<FA, FB, OF>(a, lda, xa, ld_xa, b, ldb, b_group_stride, xb, ld_xb, xb_group_stride, offsets, g, \
                                 total_m, n, k, d, ldd, st)
#define BY_OUT(FA, FB) return out_f32 ? CALL(FA, FB, true) : CALL(FA, FB, false)
    if (fa == kE4M3 && fb == kE4M3) BY_OUT(kE4M3, kE4M3);
    if (fa == kE4M3 && fb == kE5M2) BY_OUT(kE4M3, kE5M2);
    if (fa == kE5M2 && fb == kE4M3) BY_OUT(kE5M2, kE4M3);
    BY_OUT(kE5M2, kE5M2);
#undef BY_OUT
#undef CALL
}

// fnuz operands (any pair with at least one fnuz format): the bf16 compatibility kernels.
template <int FA, int FB, bool OUT_F32>
hipError_t compat_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                        const float* sa, int sa_vec, const float* sb, int sb_vec, void* d, int64_t ldd,
                        hipStream_t st) {
    const int64_t tiles = ((m + compat::BM - 1) / compat::BM) * ((n + compat::BN - 1) / compat::BN);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gemm_compat<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, st, a, lda, b, ldb,
                       m, n, k, sa, sa_vec, sb, sb_vec, d, ldd);
    return hipGetLastError();
}

template <int FA, int FB, bool OUT_F32>
hipError_t grouped_compat_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t stride,
                                const int64_t* offsets, int g, int64_t total_m, int64_t n, int64_t k, const float* sa,
                                const float* sb, void* d, int64_t ldd, hipStream_t st) {
    if (total_m == 0 || n == 0) return hipSuccess;
    const int64_t tiles = ((total_m + compat::BM - 1) / compat::BM + g) * ((n + compat::BN - 1) / compat::BN);
    hipLaunchKernelGGL((k_grouped_gemm_compat<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, st, a, lda,
                       b, ldb, stride, offsets, g, total_m, n, k, sa, sb, d, ldd);
    return hipGetLastError();
}

// Dispatch over the 16 format pairs of the compatibility kernels.
#define FP8_COMPAT_PAIRS(CALL)                                  \
    switch (fa * 4 + fb) {                                      \
        case 0: return CALL(kE4M3, kE4M3);                      \
        case 1: return CALL(kE4M3, kE5M2);                      \
        case 2: return CALL(kE4M3, kE4M3Fnuz);                  \
        case 3: return CALL(kE4M3, kE5M2Fnuz);                  \
        case 4: return CALL(kE5M2, kE4M3);                      \
        case 5: return CALL(kE5M2, kE5M2);                      \
        case 6: return CALL(kE5M2, kE4M3Fnuz);                  \
        case 7: return CALL(kE5M2, kE5M2Fnuz);                  \
        case 8: return CALL(kE4M3Fnuz, kE4M3);                  \
        case 9: return CALL(kE4M3Fnuz, kE5M2);                  \
        case 10: return CALL(kE4M3Fnuz, kE4M3Fnuz);             \
        case 11: return CALL(kE4M3Fnuz, kE5M2Fnuz);             \
        case 12: return CALL(kE5M2Fnuz, kE4M3);                 \
        case 13: return CALL(kE5M2Fnuz, kE5M2);                 \
        case 14: return CALL(kE5M2Fnuz, kE4M3Fnuz);             \
        default: return CALL(kE5M2Fnuz, kE5M2Fnuz);             \
    }

hipError_t launch_gemm_compat(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t m,
                              int64_t n, int64_t k, const float* sa, int sa_vec, const float* sb, int sb_vec, void* d,
                              int out_f32, int64_t ldd, hipStream_t st) {
#define CALL(FA, FB)                                                                                            \
    (out_f32 ? compat_typed<FA, FB, true>(a, lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, st)         \
             : compat_typed<FA, FB, false>(a, lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, st))
    FP8_COMPAT_PAIRS(CALL)
#undef CALL
}

hipError_t launch_grouped_gemm_compat(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                                      int64_t b_group_stride, const int64_t* offsets, int g, int64_t total_m,
                                      int64_t n, int64_t k, const float* sa, const float* sb, void* d, int out_f32,
                                      int64_t ldd, hipStream_t st) {
#define CALL(FA, FB)                                                                                               \
    (out_f32 ? grouped_compat_typed<FA, FB, true>(a, lda, b, ldb, b_group_stride, offsets, g, total_m, n, k, sa, sb, \
                                                  d, ldd, st)                                                      \
             : grouped_compat_typed<FA, FB, false>(a, lda, b, ldb, b_group_stride, offsets, g, total_m, n, k, sa, sb, \
                                                   d, ldd, st))
    FP8_COMPAT_PAIRS(CALL)
#undef CALL
}
#undef FP8_COMPAT_PAIRS

hipError_t launch_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t m,
                       int64_t n, int64_t k, const float* sa, int sa_vec, const float* sb, int sb_vec, void* d,
                       int out_f32, int64_t ldd, hipStream_t st) {
#define CALL(FA, FB, OF) gemm_typed<FA, FB, OF>(a, lda, b, ldb, m, n, k, sa, sa_vec, sb, sb_vec, d, ldd, st)
#define BY_OUT(FA, FB) return out_f32 ? CALL(FA, FB, true) : CALL(FA, FB, false)
    if (fa == kE4M3 && fb == kE4M3) BY_OUT(kE4M3, kE4M3);
    if (fa == kE4M3 && fb == kE5M2) BY_OUT(kE4M3, kE5M2);
    if (fa == kE5M2 && fb == kE4M3) BY_OUT(kE5M2, kE4M3);
    BY_OUT(kE5M2, kE5M2);
#undef BY_OUT
#undef CALL
}

hipError_t launch_grouped_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                               int64_t b_group_stride, const int64_t* offsets, int g, int64_t total_m, int64_t n,
                               int64_t k, const float* sa, const float* sb, void* d, int out_f32, int64_t ldd,
                               hipStream_t st) {
#define CALL(FA, FB, OF) \
    grouped_typed<FA, FB, OF>(a, lda, b, ldb, b_group_stride, offsets, g, total_m, n, k, sa, sb, d, ldd, st)
#define BY_OUT(FA, FB) return out_f32 ? CALL(FA, FB, true) : CALL(FA, FB, false)
    if (fa == kE4M3 && fb == kE4M3) BY_OUT(kE4M3, kE4M3);
    if (fa == kE4M3 && fb == kE5M2) BY_OUT(kE4M3, kE5M2);
    if (fa == kE5M2 && fb == kE4M3) BY_OUT(kE5M2, kE4M3);
    BY_OUT(kE5M2, kE5M2);
#undef BY_OUT
#undef CALL
}

}  // namespace fp8amax
