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
// Large-tile kernel: 256 x 256 x 128 per workgroup, one 128 x 128 quadrant per
// wavefront (4 x 4 blocks of 32x32x64, 256 fp32 accumulators per lane), two
// LDS stages filled by direct global->LDS loads (global_load_lds_dwordx4: each
// lane's 16 bytes land at stage base + 16 * lane, so the XOR swizzle of the
// LDS layout is produced by choosing which global chunk each lane fetches).
// Requires k % 128 == 0 (no K tail); rows past m / n are clamped to the last
// valid row on load and never stored.
namespace big {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int kStage = (BM + BN) * BK;              // 64 KB: A tile then B tile
constexpr int kEpiPitch = 256 + 16;                 // bytes per staged bf16 output row (128 cols + pad)
constexpr int kEpiWave = 128 * kEpiPitch;           // one wavefront's 128 x 128 bf16 block
constexpr int kSmem = 4 * kEpiWave > 2 * kStage ? 4 * kEpiWave : 2 * kStage;
}  // namespace big

typedef __attribute__((address_space(3))) void lds_void;

// Issue this thread's share of one stage: A rows [0, 256) and B rows [0, 256)
// of the K slice starting at k0. Wave w, instruction i fills LDS row group
// g = w*8 + i (8 rows of 128 bytes); lane l fills row 8g + l/8, slot l%8,
// which holds K chunk (l%8) ^ (row & 7).
__device__ __forceinline__ void big_issue_stage(uint8_t* stage, const uint8_t* a, int64_t lda, int64_t a_rows,
                                                const uint8_t* b, int64_t ldb, int64_t b_rows, int64_t k0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane >> 3;
    const int chunk = (lane & 7) ^ rl;                  // row & 7 == rl for rows 8g + rl
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int g = wave * 8 + i;
        int64_t r = g * 8 + rl;
        r = r < a_rows ? r : a_rows - 1;
        __builtin_amdgcn_global_load_lds(a + r * lda + k0 + chunk * 16, (lds_void*)(stage + g * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int g = wave * 8 + i;
        int64_t r = g * 8 + rl;
        r = r < b_rows ? r : b_rows - 1;
        __builtin_amdgcn_global_load_lds(b + r * ldb + k0 + chunk * 16, (lds_void*)(stage + big::BM * big::BK + g * 1024),
                                         16, 0, 0);
    }
}

__device__ __forceinline__ v8i big_frag(const uint8_t* tile, int row, int kk) {
    const int lane = threadIdx.x & 63;
    const int c0 = kk * 4 + (lane >> 5) * 2;
    const uint8_t* rp = tile + row * 128;
    const uint4 lo = *reinterpret_cast<const uint4*>(rp + ((c0 ^ (row & 7)) << 4));
    const uint4 hi = *reinterpret_cast<const uint4*>(rp + (((c0 + 1) ^ (row & 7)) << 4));
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
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

template <int FA, int FB>
__device__ __forceinline__ void big_mainloop(uint8_t* smem, const uint8_t* a, int64_t lda, int64_t a_rows,
                                             const uint8_t* b, int64_t ldb, int64_t b_rows, int64_t k,
                                             v16f (&acc)[4][4]) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;
    const int64_t nk = k / big::BK;
    big_issue_stage(smem, a, lda, a_rows, b, ldb, b_rows, 0);
    for (int64_t kt = 0; kt < nk; ++kt) {
        uint8_t* cur = smem + (kt & 1) * big::kStage;
        // this stage's loads have landed for every wavefront
        __builtin_amdgcn_s_waitcnt(0x0f70);             // vmcnt(0)
        __syncthreads();
        if (kt + 1 < nk)
            big_issue_stage(smem + ((kt + 1) & 1) * big::kStage, a, lda, a_rows, b, ldb, b_rows, (kt + 1) * big::BK);
        const uint8_t* As = cur;
        const uint8_t* Bs = cur + big::BM * big::BK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i fa[4], fb[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) fa[mi] = big_frag(As, wm * 128 + mi * 32 + (lane & 31), kk);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) fb[ni] = big_frag(Bs, wn * 128 + ni * 32 + (lane & 31), kk);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[mi], fb[ni], acc[mi][ni], MfmaFmt<FA>::v, MfmaFmt<FB>::v, 0, 0, 0, 0);
        }
        // the next iteration's barrier also guarantees every wavefront is done
        // reading this stage before it is refilled two iterations later
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
    v16f acc[4][4];
    big_mainloop<FA, FB>(smem, a + row0 * lda, lda, m - row0, b + col0 * ldb, ldb, n - col0, k, acc);

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t wrow0 = row0 + wm * 128, wcol0 = col0 + wn * 128;
    const int64_t rows_valid = m - wrow0, cols_valid = n - wcol0;
    float sbj[4];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
        int64_t j = ni * 32 + (lane & 31);
        j = j < cols_valid ? j : cols_valid - 1;
        sbj[ni] = sb[sb_vec ? (cols_valid > 0 ? wcol0 + j : 0) : 0];
    }
    if (OUT_F32 || !vec_out) {
        // direct stores from registers
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lr = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (lr >= rows_valid) continue;
                const float sai = sa[sa_vec ? wrow0 + lr : 0];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const int lc = ni * 32 + (lane & 31);
                    if (lc >= cols_valid) continue;
                    const float v = acc[mi][ni][r] * sai * sbj[ni];
                    const int64_t off = (wrow0 + lr) * ldd + wcol0 + lc;
                    if (OUT_F32)
                        reinterpret_cast<float*>(d)[off] = v;
                    else
                        reinterpret_cast<uint16_t*>(d)[off] = (uint16_t)f32_to_bf16(v);
                }
            }
        return;
    }
    // bf16 through LDS: each wavefront stages its 128 x 128 block row-major
    // (padded rows), then streams it out 16 bytes per lane, 4 rows of 256
    // contiguous bytes per store instruction.
    __syncthreads();                                     // all wavefronts are done with the stages
    uint8_t* ep = smem + wave * big::kEpiWave;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int lr = mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            int64_t gr = lr < rows_valid ? wrow0 + lr : (rows_valid > 0 ? wrow0 + rows_valid - 1 : wrow0);
            const float sai = sa[sa_vec ? gr : 0];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const int lc = ni * 32 + (lane & 31);
                const float v = acc[mi][ni][r] * sai * sbj[ni];
                *reinterpret_cast<uint16_t*>(ep + lr * big::kEpiPitch + lc * 2) = (uint16_t)f32_to_bf16(v);
            }
        }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
        const int lr = it * 4 + (lane >> 4);
        const int ch = lane & 15;                        // 8 bf16 columns
        if (lr >= rows_valid) continue;
        const uint4 val = *reinterpret_cast<const uint4*>(ep + lr * big::kEpiPitch + ch * 16);
        uint16_t* dst = reinterpret_cast<uint16_t*>(d) + (wrow0 + lr) * ldd + wcol0 + ch * 8;
        if (ch * 8 + 8 <= cols_valid) {
            *reinterpret_cast<uint4*>(dst) = val;
        } else {
            const uint32_t w[4] = {val.x, val.y, val.z, val.w};
            for (int e = 0; e < 8 && ch * 8 + e < cols_valid; ++e) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

template <int FA, int FB, bool OUT_F32>
hipError_t gemm_typed(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb, int64_t m, int64_t n, int64_t k,
                      const float* sa, int sa_vec, const float* sb, int sb_vec, void* d, int64_t ldd,
                      hipStream_t st) {
    const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    const int64_t big_tiles = ((m + big::BM - 1) / big::BM) * ((n + big::BN - 1) / big::BN);
    if (k > 0 && k % big::BK == 0 && big_tiles >= 128) {
        const int vec_out = (reinterpret_cast<uintptr_t>(d) % 16 == 0) && ldd % 8 == 0;
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
    hipLaunchKernelGGL((k_grouped_gemm<FA, FB, OUT_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, st, a, lda, b, ldb,
                       stride, offsets, g, total_m, n, k, sa, sb, d, ldd);
    return hipGetLastError();
}

}  // namespace

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
