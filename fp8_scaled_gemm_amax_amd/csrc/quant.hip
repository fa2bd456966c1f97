// quant.hip - memory-bound FP8 kernels for gfx950: amax reductions, the fused
// rowwise / tensorwise amax+scale+cast quantizers, the colwise quantizer with a
// transposed, coalesced output, and the fused delayed-scale update.
//
// Sources: "FP8 Training on AMD GPUs with TorchTitan and TorchAO" (fused
// quantization kernels replacing a chain of eager kernels; the colwise-scales
// kernel whose non-coalesced writes cost the MoE layer); "FP8 training for Flux
// models", section "Configuration" (delayed/tensorwise recipes, history length,
// compute algo, margin) and section "Testing" (fused delayed-scale update).
//
// Layout choices for CDNA4: one 64-lane wavefront per row for row reductions
// (the reduction stays inside the wavefront: no LDS, no barrier), 16-byte
// loads of 8 bf16 per lane, 8-byte stores of 8 codes per lane, amax on packed
// 16-bit magnitude bits (two elements per instruction), cross-workgroup
// combination by one relaxed atomic max per workgroup.
#include "fp8_device.hpp"
#include "kernels.hpp"

namespace fp8amax {

namespace {

constexpr int kBlock = 256;   // 4 wavefronts
constexpr int kWaves = kBlock / 64;

template <int F>
__device__ __forceinline__ uint32_t encode1(float v) {
    return encode_sw<F>(v);
}

__device__ __forceinline__ uint32_t word_absmax(uint32_t acc, uint4 v) {
    acc = pk_absmax(acc, v.x);
    acc = pk_absmax(acc, v.y);
    acc = pk_absmax(acc, v.z);
    return pk_absmax(acc, v.w);
}

// Eight bf16 values (one 16-byte chunk) times s -> eight codes.
template <int F, bool NAN_FREE>
__device__ __forceinline__ uint2 encode8(uint4 v, float s) {
    uint2 o;
    o.x = encode4<F, NAN_FREE>(bf16_lo(v.x) * s, bf16_hi(v.x) * s, bf16_lo(v.y) * s, bf16_hi(v.y) * s);
    o.y = encode4<F, NAN_FREE>(bf16_lo(v.z) * s, bf16_hi(v.z) * s, bf16_lo(v.w) * s, bf16_hi(v.w) * s);
    return o;
}

// Block-wide max of per-lane magnitude bits (32-bit); result valid in all threads.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    uint32_t r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = lds[w] > r ? lds[w] : r;
    return r;
}

// ----------------------------------------------------------------------- fill --

__global__ void k_fill(float* __restrict__ p, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// ----------------------------------------------------------------------- amax --

// Row amax, one wavefront per row. VEC: 16-byte loads (x aligned, ldx % 8 == 0,
// cols % 8 == 0); otherwise element loads.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_amax_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t ldx, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    uint32_t mx = 0;
    if (VEC) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
        const int64_t nch = cols >> 3;
        for (int64_t c = lane; c < nch; c += 64) mx = word_absmax(mx, xr[c]);
        mx = pk_fold(mx);
    } else {
        const uint16_t* xr = x + row * ldx;
        for (int64_t c = lane; c < cols; c += 64) {
            uint32_t b = xr[c] & 0x7fffu;
            mx = b > mx ? b : mx;
        }
    }
    mx = wave_max_u32(mx);
    if (lane == 0) out[row] = amax_from_bits16(mx);
}

// Column amax: a workgroup covers 512 columns (64 lanes x 8) of a band of
// kColRows rows, four rows at a time (one per wavefront); partial maxima meet
// in LDS and each column is folded into out[] by one atomic max (out cleared
// beforehand).
constexpr int kColRows = 256;

__global__ __launch_bounds__(kBlock) void k_amax_cols_vec(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, float* __restrict__ out) {
    __shared__ uint32_t part[kWaves][256];   // packed u16 pairs: 512 columns
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ch = (int64_t)blockIdx.x * 64 + lane;        // 8-column chunk index
    const int64_t nch = cols >> 3;
    const int64_t r0 = (int64_t)blockIdx.y * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    if (ch < nch) {
        const uint16_t* base = x + ch * 8;
        int64_t r = r0 + wave;
        for (; r + 3 * kWaves < r1; r += 4 * kWaves) {
            uint4 v0 = *reinterpret_cast<const uint4*>(base + r * ldx);
            uint4 v1 = *reinterpret_cast<const uint4*>(base + (r + kWaves) * ldx);
            uint4 v2 = *reinterpret_cast<const uint4*>(base + (r + 2 * kWaves) * ldx);
            uint4 v3 = *reinterpret_cast<const uint4*>(base + (r + 3 * kWaves) * ldx);
            m0 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m0, v0.x), v1.x), v2.x), v3.x);
            m1 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m1, v0.y), v1.y), v2.y), v3.y);
            m2 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m2, v0.z), v1.z), v2.z), v3.z);
            m3 = pk_absmax(pk_absmax(pk_absmax(pk_absmax(m3, v0.w), v1.w), v2.w), v3.w);
        }
        for (; r < r1; r += kWaves) {
            uint4 v = *reinterpret_cast<const uint4*>(base + r * ldx);
            m0 = pk_absmax(m0, v.x);
            m1 = pk_absmax(m1, v.y);
            m2 = pk_absmax(m2, v.z);
            m3 = pk_absmax(m3, v.w);
        }
    }
    part[wave][lane * 4 + 0] = m0;
    part[wave][lane * 4 + 1] = m1;
    part[wave][lane * 4 + 2] = m2;
    part[wave][lane * 4 + 3] = m3;
    __syncthreads();
    // thread t folds word t (two columns) over the four wavefronts
    const int t = threadIdx.x;
    uint32_t w = part[0][t];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) w = pk_absmax(w, part[k][t]);
    const int64_t col = (int64_t)blockIdx.x * 512 + 2 * t;
    if (col < cols) atomic_max_bits(out + col, (w & 0xffffu) << 16);
    if (col + 1 < cols) atomic_max_bits(out + col + 1, w & 0xffff0000u);
}

__global__ __launch_bounds__(kBlock) void k_amax_cols_scalar(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx, float* __restrict__ out) {
    const int64_t col = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (col >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.y * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    uint32_t mx = 0;
    for (int64_t r = r0; r < r1; ++r) {
        uint32_t b = x[r * ldx + col] & 0x7fffu;
        mx = b > mx ? b : mx;
    }
    atomic_max_bits(out + col, mx << 16);
}

// Whole-tensor amax: wavefronts stride over rows; one atomic max per workgroup.
template <bool VEC>
__global__ __launch_bounds__(kBlock) void k_amax_tensor(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                        int64_t ldx, float* __restrict__ out) {
    __shared__ uint32_t red[kWaves];
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    uint32_t mx = 0;
    for (int64_t row = wave_id; row < rows; row += nwaves) {
        if (VEC) {
            const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
            const int64_t nch = cols >> 3;
            for (int64_t c = lane; c < nch; c += 64) mx = word_absmax(mx, xr[c]);
        } else {
            const uint16_t* xr = x + row * ldx;
            for (int64_t c = lane; c < cols; c += 64) {
                uint32_t b = xr[c] & 0x7fffu;
                mx = b > mx ? b : mx;
            }
        }
    }
    if (VEC) mx = pk_fold(mx);
    mx = block_max_u32(mx, red);
    if (threadIdx.x == 0) atomic_max_bits(out, mx << 16);
}

// ---------------------------------------------------------- rowwise quantizer --

// One wavefront per row, the whole row held in registers (MAXC 16-byte chunks
// per lane): read once, amax, scale, cast, write once.
template <int F, int MAXC>
__global__ __launch_bounds__(kBlock) void k_quant_row_reg(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, int margin, uint8_t* __restrict__ q,
                                                          int64_t ldq, float* __restrict__ scale_inv,
                                                          float* __restrict__ amax_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nch = (int)(cols >> 3);
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = ch < nch ? xr[ch] : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) mx = word_absmax(mx, v[c]);
    const float amax = amax_from_bits16(wave_max_u32(pk_fold(mx)));
    const float s = scale_from_amax<F>(amax, margin);
    if (lane == 0) {
        scale_inv[row] = 1.0f / s;
        if (amax_out) amax_out[row] = amax;
    }
    uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
    if (!__builtin_isnan(amax)) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            if (ch < nch) qr[ch] = encode8<F, true>(v[c], s);
        }
    } else {   // a NaN in the row (then s = 1): the bit-level encoder keeps NaN signs
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            if (ch < nch) qr[ch] = encode8<F, false>(v[c], s);
        }
    }
}

// Rows too long for registers, or unaligned layouts: two passes over the row
// (the second pass hits in cache).
template <int F, bool VEC>
__global__ __launch_bounds__(kBlock) void k_quant_row_2pass(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, int margin,
                                                            uint8_t* __restrict__ q, int64_t ldq,
                                                            float* __restrict__ scale_inv,
                                                            float* __restrict__ amax_out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t* xr = x + row * ldx;
    uint8_t* qr = q + row * ldq;
    uint32_t mx = 0;
    if (VEC) {
        const int64_t nch = cols >> 3;
        for (int64_t c = lane; c < nch; c += 64) mx = word_absmax(mx, reinterpret_cast<const uint4*>(xr)[c]);
        mx = pk_fold(mx);
    } else {
        for (int64_t c = lane; c < cols; c += 64) {
            uint32_t b = xr[c] & 0x7fffu;
            mx = b > mx ? b : mx;
        }
    }
    const float amax = amax_from_bits16(wave_max_u32(mx));
    const float s = scale_from_amax<F>(amax, margin);
    if (lane == 0) {
        scale_inv[row] = 1.0f / s;
        if (amax_out) amax_out[row] = amax;
    }
    if (VEC) {
        const int64_t nch = cols >> 3;
        if (!__builtin_isnan(amax)) {
            for (int64_t c = lane; c < nch; c += 64)
                reinterpret_cast<uint2*>(qr)[c] = encode8<F, true>(reinterpret_cast<const uint4*>(xr)[c], s);
        } else {
            for (int64_t c = lane; c < nch; c += 64)
                reinterpret_cast<uint2*>(qr)[c] = encode8<F, false>(reinterpret_cast<const uint4*>(xr)[c], s);
        }
    } else {
        for (int64_t c = lane; c < cols; c += 64) qr[c] = (uint8_t)encode1<F>(bf16_lo(xr[c]) * s);
    }
}

// ------------------------------------------------------- tensorwise quantizer --

// Cast with one scale: DELAYED reads the scale from the state and folds the
// tensor's amax into amax_io; otherwise the scale comes from amax_io (the
// amax pass already ran). Wavefronts stride over rows.
template <int F, bool VEC, bool DELAYED>
__global__ __launch_bounds__(kBlock) void k_quant_tensor(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ldx, int margin, const float* __restrict__ scale,
                                                         uint8_t* __restrict__ q, int64_t ldq,
                                                         float* __restrict__ scale_inv, float* __restrict__ amax_io) {
    __shared__ uint32_t red[kWaves];
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const float s = DELAYED ? *scale : scale_from_amax<F>(*amax_io, margin);
    const bool tensor_nan = DELAYED ? false : __builtin_isnan(*amax_io);
    if (blockIdx.x == 0 && threadIdx.x == 0) scale_inv[0] = 1.0f / s;
    uint32_t mx = 0;
    for (int64_t row = wave_id; row < rows; row += nwaves) {
        const uint16_t* xr = x + row * ldx;
        uint8_t* qr = q + row * ldq;
        if (VEC) {
            const int64_t nch = cols >> 3;
            for (int64_t c = lane; c < nch; c += 64) {
                const uint4 v = reinterpret_cast<const uint4*>(xr)[c];
                // NaN check: the running max of this lane turns NaN with the
                // first NaN it sees (without the delayed amax, the tensor's
                // amax from the first pass decides for the whole tensor)
                bool nan_seen;
                if (DELAYED) {
                    mx = word_absmax(mx, v);
                    nan_seen = nan_bits16(pk_fold(mx));
                } else {
                    nan_seen = tensor_nan;
                }
                reinterpret_cast<uint2*>(qr)[c] = nan_seen ? encode8<F, false>(v, s) : encode8<F, true>(v, s);
            }
        } else {
            for (int64_t c = lane; c < cols; c += 64) {
                const uint32_t b = xr[c];
                if (DELAYED) mx = (b & 0x7fffu) > mx ? (b & 0x7fffu) : mx;
                qr[c] = (uint8_t)encode1<F>(bf16_lo(b) * s);
            }
        }
    }
    if (DELAYED) {
        if (VEC) mx = pk_fold(mx);
        mx = block_max_u32(mx, red);
        if (threadIdx.x == 0) atomic_max_bits(amax_io, mx << 16);
    }
}

// ---------------------------------------------------------- colwise quantizer --

// Scales of the workgroup's 64 columns, computed once into LDS.
template <int F>
__device__ __forceinline__ void col_scales_to_lds(const float* __restrict__ col_amax, int64_t c0, int64_t cols,
                                                  int margin, float* __restrict__ scale_inv, float* s_lds,
                                                  int* nan_lds) {
    if (threadIdx.x < 64) {
        const int64_t c = c0 + threadIdx.x;
        const float a = c < cols ? col_amax[c] : 0.0f;
        const float s = scale_from_amax<F>(a, margin);
        s_lds[threadIdx.x] = s;
        nan_lds[threadIdx.x] = __builtin_isnan(a) ? 1 : 0;
        if (blockIdx.y == 0 && c < cols) scale_inv[c] = 1.0f / s;
    }
    __syncthreads();
}

// Transposed colwise cast through LDS. A workgroup owns a tile of 128 rows x 64
// columns. Read: lane (cc = t % 8, rg = t / 8) loads rows 4rg..4rg+3 of
// columns 8cc..8cc+7 (each row segment of the tile is one 128-byte line),
// casts with the column scales, and transposes its two 4x4 byte blocks in
// registers (byte permutes), so that each 32-bit word holds four consecutive
// rows of one column. The words go to LDS laid out [column][128 rows] with the
// 16-byte row-chunk index XOR-swizzled by the column's chunk group (spreads
// the 64 lanes' writes over banks). Write: 8 lanes stream one output row
// (= input column) as 128 contiguous bytes.
constexpr int kColTileR = 128, kColTileC = 64;

template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_col_tiled(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, int margin,
                                                            uint8_t* __restrict__ qt, int64_t ldqt,
                                                            float* __restrict__ scale_inv,
                                                            const float* __restrict__ col_amax, int vec_store) {
    __shared__ float s_lds[kColTileC];
    __shared__ int nan_lds[kColTileC];
    __shared__ __attribute__((aligned(16))) uint32_t tile[kColTileC * kColTileR / 4];
    const int64_t c0 = (int64_t)blockIdx.x * kColTileC;
    const int64_t r0 = (int64_t)blockIdx.y * kColTileR;
    col_scales_to_lds<F>(col_amax, c0, cols, margin, scale_inv, s_lds, nan_lds);

    const int t = threadIdx.x;
    const int cc = t & 7, rg = t >> 3;
    const int64_t col = c0 + cc * 8;
    uint32_t w[4][2];
    float s[8];
    int any_nan = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s[j] = s_lds[cc * 8 + j];
        any_nan |= nan_lds[cc * 8 + j];
    }
    uint4 v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + rg * 4 + r;
        v[r] = make_uint4(0u, 0u, 0u, 0u);
        if (row < rows && col < cols) v[r] = *reinterpret_cast<const uint4*>(x + row * ldx + col);
    }
    if (!any_nan) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w[r][0] = encode4<F, true>(bf16_lo(v[r].x) * s[0], bf16_hi(v[r].x) * s[1], bf16_lo(v[r].y) * s[2],
                                       bf16_hi(v[r].y) * s[3]);
            w[r][1] = encode4<F, true>(bf16_lo(v[r].z) * s[4], bf16_hi(v[r].z) * s[5], bf16_lo(v[r].w) * s[6],
                                       bf16_hi(v[r].w) * s[7]);
        }
    } else {   // a column of this chunk holds a NaN: bit-level encoder
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w[r][0] = encode4<F, false>(bf16_lo(v[r].x) * s[0], bf16_hi(v[r].x) * s[1], bf16_lo(v[r].y) * s[2],
                                        bf16_hi(v[r].y) * s[3]);
            w[r][1] = encode4<F, false>(bf16_lo(v[r].z) * s[4], bf16_hi(v[r].z) * s[5], bf16_lo(v[r].w) * s[6],
                                        bf16_hi(v[r].w) * s[7]);
        }
    }
    const int chunk = ((rg >> 2) ^ cc) & 7;       // swizzled 16-byte row chunk
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        // 4x4 byte transpose: rows r = 0..3 (words) x columns c = 0..3 (bytes)
        const uint32_t a_lo = __builtin_amdgcn_perm(w[1][h], w[0][h], 0x05010400u);
        const uint32_t a_hi = __builtin_amdgcn_perm(w[1][h], w[0][h], 0x07030602u);
        const uint32_t b_lo = __builtin_amdgcn_perm(w[3][h], w[2][h], 0x05010400u);
        const uint32_t b_hi = __builtin_amdgcn_perm(w[3][h], w[2][h], 0x07030602u);
        const uint32_t tcol[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u),
                                  __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                                  __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u),
                                  __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int lc = cc * 8 + h * 4 + c;     // local column
            tile[lc * (kColTileR / 4) + chunk * 4 + (rg & 3)] = tcol[c];
        }
    }
    __syncthreads();
    // 64 columns x 8 chunks of 16 bytes; two per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = t + i * kBlock;
        const int lc = p >> 3, rc = p & 7;
        const int64_t ocol = c0 + lc;
        if (ocol >= cols) continue;
        const int sw = (rc ^ (lc >> 3)) & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(&tile[lc * (kColTileR / 4) + sw * 4]);
        const int64_t orow = r0 + rc * 16;
        uint8_t* dst = qt + ocol * ldqt + orow;
        if (vec_store && orow + 16 <= rows) {
            *reinterpret_cast<uint4*>(dst) = val;
        } else {
            const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
            for (int b = 0; b < 16 && orow + b < rows; ++b) dst[b] = (uint8_t)(wv[b >> 2] >> (8 * (b & 3)));
        }
    }
}

// Any layout: one thread per column of a band of rows (reads coalesce across
// threads, writes do not; this path is for layouts the tiled kernel rejects).
template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_col_scalar(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx, int margin,
                                                             uint8_t* __restrict__ qt, int64_t ldqt,
                                                             float* __restrict__ scale_inv,
                                                             const float* __restrict__ col_amax) {
    const int64_t col = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (col >= cols) return;
    const float s = scale_from_amax<F>(col_amax[col], margin);
    if (blockIdx.y == 0) scale_inv[col] = 1.0f / s;
    const int64_t r0 = (int64_t)blockIdx.y * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    for (int64_t r = r0; r < r1; ++r) qt[col * ldqt + r] = (uint8_t)encode1<F>(bf16_lo(x[r * ldx + col]) * s);
}

// ------------------------------------------------------ delayed scale update --

// One wavefront per tensor. The effective amax combines the value being
// recorded with the other L-1 ring slots (the slot at head is the one being
// overwritten), so no lane reads a slot another lane is writing.
template <int F>
__global__ __launch_bounds__(kBlock) void k_delayed_update(float* __restrict__ cur_amax, float* __restrict__ history,
                                                           const int32_t* __restrict__ head, int64_t n, int L,
                                                           int algo, int margin, float* __restrict__ scale,
                                                           float* __restrict__ scale_inv) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (i >= n) return;
    const int h = ((*head % L) + L) % L;     // a corrupt head cannot index outside the ring
    const float cur = cur_amax[i];
    float* hist = history + i * (int64_t)L;
    uint32_t mx = __float_as_uint(cur) & 0x7fffffffu;
    if (algo == 1) {
        for (int t = lane; t < L; t += 64) {
            if (t == h) continue;
            const uint32_t b = __float_as_uint(hist[t]) & 0x7fffffffu;
            mx = b > mx ? b : mx;
        }
        mx = wave_max_u32(mx);
    }
    if (lane == 0) {
        hist[h] = cur;
        float s;
        if (delayed_scale<F>(__uint_as_float(mx), margin, &s)) {
            scale[i] = s;
            scale_inv[i] = 1.0f / s;
        }
        cur_amax[i] = 0.0f;
    }
}

__global__ void k_advance_head(int32_t* head, int L) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *head = (((*head % L) + L) % L + 1) % L;
}

// ------------------------------------------------------------------ helpers --

int grid_for_rows(int64_t rows) { return (int)((rows + kWaves - 1) / kWaves); }

int strided_grid(int64_t rows) {
    const int64_t cap = (int64_t)current_device_props().cus * 4;
    const int64_t need = (rows + kWaves - 1) / kWaves;
    return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

bool is_aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <int F>
hipError_t quant_row_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin, uint8_t* q,
                         int64_t ldq, float* scale_inv, float* amax_out, hipStream_t st) {
    const dim3 grid(grid_for_rows(rows)), block(kBlock);
    const bool vec = is_aligned(x, 16) && is_aligned(q, 8) && ldx % 8 == 0 && ldq % 8 == 0 && cols % 8 == 0;
    if (!vec) {
        hipLaunchKernelGGL((k_quant_row_2pass<F, false>), grid, block, 0, st, x, rows, cols, ldx, margin, q, ldq,
                           scale_inv, amax_out);
        return hipGetLastError();
    }
    const int64_t per_lane = (cols / 8 + 63) / 64;
#define FP8_ROW_CASE(C)                                                                                        \
    if (per_lane <= C) {                                                                                       \
        hipLaunchKernelGGL((k_quant_row_reg<F, C>), grid, block, 0, st, x, rows, cols, ldx, margin, q, ldq,    \
                           scale_inv, amax_out);                                                               \
        return hipGetLastError();                                                                              \
    }
    FP8_ROW_CASE(1)
    FP8_ROW_CASE(2)
    FP8_ROW_CASE(4)
    FP8_ROW_CASE(8)
    FP8_ROW_CASE(16)
    FP8_ROW_CASE(32)
#undef FP8_ROW_CASE
    hipLaunchKernelGGL((k_quant_row_2pass<F, true>), grid, block, 0, st, x, rows, cols, ldx, margin, q, ldq,
                       scale_inv, amax_out);
    return hipGetLastError();
}

template <int F>
hipError_t quant_col_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin, uint8_t* qt,
                         int64_t ldqt, float* scale_inv, const float* col_amax, hipStream_t st) {
    const bool vec_in = is_aligned(x, 16) && ldx % 8 == 0 && cols % 8 == 0;
    if (vec_in) {
        const int vec_store = is_aligned(qt, 16) && ldqt % 16 == 0;
        const dim3 grid((unsigned)((cols + kColTileC - 1) / kColTileC), (unsigned)((rows + kColTileR - 1) / kColTileR));
        hipLaunchKernelGGL((k_quant_col_tiled<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, qt, ldqt,
                           scale_inv, col_amax, vec_store);
    } else {
        const dim3 grid((unsigned)((cols + kBlock - 1) / kBlock), (unsigned)((rows + kColRows - 1) / kColRows));
        hipLaunchKernelGGL((k_quant_col_scalar<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, qt, ldqt,
                           scale_inv, col_amax);
    }
    return hipGetLastError();
}

template <int F>
hipError_t quant_tensor_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin,
                            const float* scale, uint8_t* q, int64_t ldq, float* scale_inv, float* amax,
                            hipStream_t st) {
    const bool vec = is_aligned(x, 16) && is_aligned(q, 8) && ldx % 8 == 0 && ldq % 8 == 0 && cols % 8 == 0;
    const dim3 grid(strided_grid(rows)), block(kBlock);
    if (scale) {
        if (vec)
            hipLaunchKernelGGL((k_quant_tensor<F, true, true>), grid, block, 0, st, x, rows, cols, ldx, margin, scale,
                               q, ldq, scale_inv, amax);
        else
            hipLaunchKernelGGL((k_quant_tensor<F, false, true>), grid, block, 0, st, x, rows, cols, ldx, margin,
                               scale, q, ldq, scale_inv, amax);
        return hipGetLastError();
    }
    hipError_t e = launch_amax(x, rows, cols, ldx, 0, amax, st);
    if (e != hipSuccess) return e;
    if (vec)
        hipLaunchKernelGGL((k_quant_tensor<F, true, false>), grid, block, 0, st, x, rows, cols, ldx, margin, scale, q,
                           ldq, scale_inv, amax);
    else
        hipLaunchKernelGGL((k_quant_tensor<F, false, false>), grid, block, 0, st, x, rows, cols, ldx, margin, scale,
                           q, ldq, scale_inv, amax);
    return hipGetLastError();
}

template <int F>
hipError_t delayed_fmt(float* cur_amax, float* history, int32_t* head, int64_t n, int L, int algo, int margin,
                       float* scale, float* scale_inv, hipStream_t st) {
    hipLaunchKernelGGL((k_delayed_update<F>), dim3(grid_for_rows(n)), dim3(kBlock), 0, st, cur_amax, history, head, n,
                       L, algo, margin, scale, scale_inv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_advance_head, dim3(1), dim3(64), 0, st, head, L);
    return hipGetLastError();
}

}  // namespace

// -------------------------------------------------------------- launchers --

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(kBlock), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis, float* out,
                       hipStream_t st) {
    const bool vec = is_aligned(x, 16) && ldx % 8 == 0 && cols % 8 == 0;
    if (axis == 1) {
        if (rows == 0) return hipSuccess;
        if (vec)
            hipLaunchKernelGGL((k_amax_rows<true>), dim3(grid_for_rows(rows)), dim3(kBlock), 0, st, x, rows, cols, ldx,
                               out);
        else
            hipLaunchKernelGGL((k_amax_rows<false>), dim3(grid_for_rows(rows)), dim3(kBlock), 0, st, x, rows, cols,
                               ldx, out);
        return hipGetLastError();
    }
    const int64_t nout = axis == 0 ? 1 : cols;
    hipError_t e = launch_fill(out, nout, 0.0f, st);
    if (e != hipSuccess || rows == 0 || cols == 0) return e;
    if (axis == 0) {
        if (vec)
            hipLaunchKernelGGL((k_amax_tensor<true>), dim3(strided_grid(rows)), dim3(kBlock), 0, st, x, rows, cols, ldx,
                               out);
        else
            hipLaunchKernelGGL((k_amax_tensor<false>), dim3(strided_grid(rows)), dim3(kBlock), 0, st, x, rows, cols,
                               ldx, out);
        return hipGetLastError();
    }
    const unsigned gy = (unsigned)((rows + kColRows - 1) / kColRows);
    if (vec)
        hipLaunchKernelGGL(k_amax_cols_vec, dim3((unsigned)((cols + 511) / 512), gy), dim3(kBlock), 0, st, x, rows,
                           cols, ldx, out);
    else
        hipLaunchKernelGGL(k_amax_cols_scalar, dim3((unsigned)((cols + kBlock - 1) / kBlock), gy), dim3(kBlock), 0, st,
                           x, rows, cols, ldx, out);
    return hipGetLastError();
}

hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            uint8_t* q, int64_t ldq, float* scale_inv, float* amax_out, hipStream_t st) {
    if (rows == 0) return hipSuccess;
#define CALL(F) quant_row_fmt<F>(x, rows, cols, ldx, margin, q, ldq, scale_inv, amax_out, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

hipError_t launch_quant_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            uint8_t* qt, int64_t ldqt, float* scale_inv, const float* col_amax, hipStream_t st) {
    if (cols == 0) return hipSuccess;
    if (rows == 0) {
        // no rows: every column has amax 0 (already in col_amax) -> scale 1
        return launch_fill(scale_inv, cols, 1.0f, st);
    }
#define CALL(F) quant_col_fmt<F>(x, rows, cols, ldx, margin, qt, ldqt, scale_inv, col_amax, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

hipError_t launch_quant_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                               const float* scale, uint8_t* q, int64_t ldq, float* scale_inv, float* amax,
                               hipStream_t st) {
#define CALL(F) quant_tensor_fmt<F>(x, rows, cols, ldx, margin, scale, q, ldq, scale_inv, amax, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

hipError_t launch_delayed_update(float* cur_amax, float* history, int32_t* head, int64_t n, int32_t L, int algo,
                                 int margin, int fmt, float* scale, float* scale_inv, hipStream_t st) {
    if (n == 0) return hipSuccess;
#define CALL(F) delayed_fmt<F>(cur_amax, history, head, n, L, algo, margin, scale, scale_inv, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

}  // namespace fp8amax
