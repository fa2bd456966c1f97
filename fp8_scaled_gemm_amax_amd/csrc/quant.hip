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

// Row amax with the row in registers (MAXC 16-byte chunks per lane, all loads
// in flight together), one wavefront per row.
template <int MAXC>
__global__ __launch_bounds__(kBlock) void k_amax_rows_reg(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nch = (int)(cols >> 3);
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));     // past the row: a duplicate chunk (a max ignores it)
    }
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) mx = word_absmax(mx, v[c]);
    mx = wave_max_u32(pk_fold(mx));
    if (lane == 0) out[row] = amax_from_bits16(mx);
}

// Column amax: a workgroup covers 512 columns (64 lanes x 8) and strides over
// bands of kColAmaxRows rows (band blockIdx.x, blockIdx.x + gridDim.x, ..; the
// grid holds about two workgroups per CU in all, so every CU gets the same
// share); wavefront w takes rows w, w + 4, .. of a band, sixteen 16-byte loads
// per lane in flight at a time. Partial maxima meet in LDS once at the end and
// each column is folded into out[] (cleared beforehand) by one atomic max per
// workgroup.
constexpr int kColRows = 256;       // row band of the scalar kernels
constexpr int kColAmaxRows = 256;   // row band of the vector column-amax kernel
constexpr int kColAmaxUnroll = 16;

__global__ __launch_bounds__(kBlock) void k_amax_cols_vec(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, float* __restrict__ out) {
    __shared__ uint32_t part[kWaves][256];   // packed u16 pairs: 512 columns
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ch = (int64_t)blockIdx.y * 64 + lane;        // 8-column chunk index
    const int64_t nch = cols >> 3;
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    if (ch < nch) {
        const uint16_t* base = x + ch * 8;
        for (int64_t r0 = (int64_t)blockIdx.x * kColAmaxRows; r0 < rows; r0 += (int64_t)gridDim.x * kColAmaxRows) {
            const int64_t r1 = r0 + kColAmaxRows < rows ? r0 + kColAmaxRows : rows;
            for (int64_t rb = r0 + wave; rb < r1; rb += kColAmaxUnroll * kWaves) {
                uint4 v[kColAmaxUnroll];
#pragma unroll
                for (int u = 0; u < kColAmaxUnroll; ++u) {
                    const int64_t r = rb + u * kWaves;
                    // rows past the band re-read its last row (a max ignores duplicates); the
                    // loads stay unconditional, so all of them are in flight together
                    v[u] = *reinterpret_cast<const uint4*>(base + (r < r1 ? r : r1 - 1) * ldx);
                }
#pragma unroll
                for (int u = 0; u < kColAmaxUnroll; ++u) {
                    m0 = pk_absmax(m0, v[u].x);
                    m1 = pk_absmax(m1, v[u].y);
                    m2 = pk_absmax(m2, v[u].z);
                    m3 = pk_absmax(m3, v[u].w);
                }
            }
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
    const int64_t col = (int64_t)blockIdx.y * 512 + 2 * t;
    if (col < cols) atomic_max_bits(out + col, (w & 0xffffu) << 16);
    if (col + 1 < cols) atomic_max_bits(out + col + 1, w & 0xffff0000u);
}

// Maxima of 16 rows across a wavefront at once: lane l holds its value of
// row u in v[u]; each exchange step pairs lanes l and l ^ o and halves the
// rows a lane carries (the lane with bit o clear keeps the lower half), so
// after the steps o = 32, 16, 8, 4 (8 + 4 + 2 + 1 shuffles) lane l carries
// row 8 b5 + 4 b4 + 2 b3 + b2 (b_i: bit i of l) over the 16 lanes that share
// bits 2..5, and two more steps (o = 2, 1) complete it: 17 shuffles instead of
// 16 full wavefront reductions. Returns that row's maximum (valid in every lane).
__device__ __forceinline__ uint32_t wave_max_16rows(const uint32_t (&v)[16]) {
    const int lane = threadIdx.x & 63;
    uint32_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool hi = lane & 32;
        const uint32_t keep = hi ? v[i + 8] : v[i], send = hi ? v[i] : v[i + 8];
        const uint32_t o = (uint32_t)__shfl_xor((int)send, 32, 64);
        a[i] = keep > o ? keep : o;
    }
    uint32_t b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bool hi = lane & 16;
        const uint32_t keep = hi ? a[i + 4] : a[i], send = hi ? a[i] : a[i + 4];
        const uint32_t o = (uint32_t)__shfl_xor((int)send, 16, 64);
        b[i] = keep > o ? keep : o;
    }
    uint32_t c[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const bool hi = lane & 8;
        const uint32_t keep = hi ? b[i + 2] : b[i], send = hi ? b[i] : b[i + 2];
        const uint32_t o = (uint32_t)__shfl_xor((int)send, 8, 64);
        c[i] = keep > o ? keep : o;
    }
    const bool hi = lane & 4;
    uint32_t d = hi ? c[1] : c[0];
    uint32_t o = (uint32_t)__shfl_xor((int)(hi ? c[0] : c[1]), 4, 64);
    d = d > o ? d : o;
    o = (uint32_t)__shfl_xor((int)d, 2, 64);
    d = d > o ? d : o;
    o = (uint32_t)__shfl_xor((int)d, 1, 64);
    return d > o ? d : o;
}

// Row and column amax in one pass (the first pass of the dual cast below):
// k_amax_cols_vec's walk, and in addition each loaded row segment's maximum
// (one wavefront covers the workgroup's 512 columns of a row) is reduced
// across the wavefront, 16 rows at a time (wave_max_16rows), and folded into
// row_out by one atomic max per row and 512-column chunk. Both outputs are
// cleared beforehand.
__global__ __launch_bounds__(kBlock) void k_amax_rows_cols_vec(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t cols, int64_t ldx, float* __restrict__ row_out,
                                                               float* __restrict__ col_out) {
    __shared__ uint32_t part[kWaves][256];   // packed u16 pairs: 512 columns
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ch = (int64_t)blockIdx.y * 64 + lane;        // 8-column chunk index
    const int64_t nch = cols >> 3;
    const bool have = ch < nch;
    const uint16_t* base = x + (have ? ch : nch - 1) * 8;      // (past the row: a duplicate chunk, not counted)
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
    for (int64_t r0 = (int64_t)blockIdx.x * kColAmaxRows; r0 < rows; r0 += (int64_t)gridDim.x * kColAmaxRows) {
        const int64_t r1 = r0 + kColAmaxRows < rows ? r0 + kColAmaxRows : rows;
        for (int64_t rb = r0 + wave; rb < r1; rb += kColAmaxUnroll * kWaves) {
            uint4 v[kColAmaxUnroll];
#pragma unroll
            for (int u = 0; u < kColAmaxUnroll; ++u) {
                const int64_t r = rb + u * kWaves;
                v[u] = *reinterpret_cast<const uint4*>(base + (r < r1 ? r : r1 - 1) * ldx);
            }
            static_assert(kColAmaxUnroll == 16, "wave_max_16rows reduces 16 rows");
            uint32_t rmax[kColAmaxUnroll];
#pragma unroll
            for (int u = 0; u < kColAmaxUnroll; ++u) {
                if (!have) v[u] = make_uint4(0u, 0u, 0u, 0u);
                m0 = pk_absmax(m0, v[u].x);
                m1 = pk_absmax(m1, v[u].y);
                m2 = pk_absmax(m2, v[u].z);
                m3 = pk_absmax(m3, v[u].w);
                rmax[u] = pk_fold(word_absmax(0u, v[u]));
            }
            const uint32_t rm = wave_max_16rows(rmax);
            const int u = ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
            const int64_t r = rb + u * kWaves;
            if ((lane & 3) == 0 && r < r1) atomic_max_bits(row_out + r, rm << 16);
        }
    }
    part[wave][lane * 4 + 0] = m0;
    part[wave][lane * 4 + 1] = m1;
    part[wave][lane * 4 + 2] = m2;
    part[wave][lane * 4 + 3] = m3;
    __syncthreads();
    const int t = threadIdx.x;
    uint32_t w = part[0][t];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) w = pk_absmax(w, part[k][t]);
    const int64_t col = (int64_t)blockIdx.y * 512 + 2 * t;
    if (col < cols) atomic_max_bits(col_out + col, (w & 0xffffu) << 16);
    if (col + 1 < cols) atomic_max_bits(col_out + col + 1, w & 0xffff0000u);
}

__global__ __launch_bounds__(kBlock) void k_amax_cols_scalar(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx, float* __restrict__ out) {
    const int64_t col = (int64_t)blockIdx.y * kBlock + threadIdx.x;
    if (col >= cols) return;
    const int64_t r0 = (int64_t)blockIdx.x * kColRows;
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

// Whole-tensor amax: wavefronts stride over rows, each row loaded whole into
// registers (MAXC 16-byte chunks per lane, all in flight at once); one atomic
// per workgroup.
template <int MAXC>
__global__ __launch_bounds__(kBlock) void k_amax_tensor_reg(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, float* __restrict__ out) {
    __shared__ uint32_t red[kWaves];
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const int nch = (int)(cols >> 3);
    uint32_t mx = 0;
    for (int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6); row < rows; row += nwaves) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
        uint4 v[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));     // past the row: a duplicate chunk, never stored
        }
#pragma unroll
        for (int c = 0; c < MAXC; ++c) mx = word_absmax(mx, v[c]);
    }
    mx = block_max_u32(pk_fold(mx), red);
    if (threadIdx.x == 0) atomic_max_bits(out, mx << 16);
}

// ---------------------------------------------------------- rowwise quantizer --

// One wavefront per row, the whole row held in registers (MAXC 16-byte chunks
// per lane): read once, amax, scale, cast, write once. NT: nontemporal loads
// (x streamed), unless another pass reads x right after.
// Codes are stored nontemporally when one launch writes more of them than the
// 256 MB last-level cache holds: kept there, they would leave it full of dirty
// lines that the consuming GEMM then has to write back while it streams its
// operands (DeepSeek-V3 expert layer: 587 MB of codes, grouped GEMM 318 ->
// 284 us). Smaller outputs stay cached for the GEMM that reads them next
// (Llama3-8B up-projection: 92 MB, where streaming them costs the GEMM 5%).
constexpr int64_t kStreamCodesAbove = (int64_t)256 << 20;
inline int streamed_codes(int64_t code_bytes) { return code_bytes > kStreamCodesAbove ? 1 : 0; }

template <int F, int MAXC, bool NT>
__device__ __forceinline__ void quant_row_one(const uint16_t* __restrict__ x, int64_t row, int64_t cols, int64_t ldx,
                                              int margin, uint8_t* __restrict__ q, int64_t ldq,
                                              float* __restrict__ scale_inv, float* __restrict__ amax_out, int nt_store) {
    const int lane = threadIdx.x & 63;
    const int nch = (int)(cols >> 3);
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = NT ? load_stream(xr + (ch < nch ? ch : nch - 1)) : xr[ch < nch ? ch : nch - 1];         // past the row: a duplicate chunk, never stored
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
            if (ch >= nch) continue;
            const uint2 code = encode8<F, true>(v[c], s);
            if (nt_store)
                __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, code),
                                            reinterpret_cast<unsigned long long*>(&qr[ch]));
            else
                qr[ch] = code;
        }
    } else {   // a NaN in the row (then s = 1): the bit-level encoder keeps NaN signs
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            if (ch < nch) qr[ch] = encode8<F, false>(v[c], s);
        }
    }
}

template <int F, int MAXC, bool NT>
__global__ __launch_bounds__(kBlock) void k_quant_row_reg(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          int64_t ldx, int margin, uint8_t* __restrict__ q,
                                                          int64_t ldq, float* __restrict__ scale_inv,
                                                          float* __restrict__ amax_out, int nt_store) {
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    quant_row_one<F, MAXC, NT>(x, row, cols, ldx, margin, q, ldq, scale_inv, amax_out, nt_store);
}

// Rowwise casts of up to kMaxRowBatch tensors with the same number of columns
// (a linear layer's activation and weight share K) in one launch: tensor j
// owns workgroups first[j] .. first[j+1]-1, one wavefront per row as above.
// One launch instead of one per tensor saves a launch gap and one ramp-up and
// drain of the memory pipeline. The arrays are indexed through compare-select
// chains on the wave-uniform tensor index (no private-memory copy).
constexpr int kMaxRowBatch = 8;
struct RowBatch {
    const uint16_t* x[kMaxRowBatch];
    uint8_t* q[kMaxRowBatch];
    float* scale_inv[kMaxRowBatch];
    float* amax[kMaxRowBatch];
    float* col_amax[kMaxRowBatch];   // column-amax side outputs (k_quant_row_colmax only; may be NULL)
    const int64_t* groups[kMaxRowBatch];   // row groups of the column amax (device offsets [ngroups + 1])
    int ngroups[kMaxRowBatch];             // 0: one column amax over all rows
    int64_t cam_first[kMaxRowBatch + 1];   // prefix sums of the column-amax sizes (k_fill_col_amax)
    int64_t rows[kMaxRowBatch];
    int64_t ldx[kMaxRowBatch];
    int64_t ldq[kMaxRowBatch];
    int64_t first[kMaxRowBatch + 1];
    int count;
    int nt_store;   // codes written nontemporally (see streamed_codes)
};

template <typename T>
__device__ __forceinline__ T batch_pick(const T (&a)[kMaxRowBatch], int j) {
    T r = a[0];
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i == j) r = a[i];
    return r;
}

template <int F, int MAXC>
__global__ __launch_bounds__(kBlock) void k_quant_row_batch(RowBatch b, int64_t cols, int margin) {
    const int64_t bid = blockIdx.x;
    // the last tensor whose first workgroup is at or before this one (an empty
    // tensor shares its start with the next, which then wins)
    int j = 0;
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i < b.count && bid >= b.first[i]) j = i;
    int64_t first = b.first[0];
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i == j) first = b.first[i];
    const int64_t row = (bid - first) * kWaves + (threadIdx.x >> 6);
    if (row >= batch_pick(b.rows, j)) return;
    quant_row_one<F, MAXC, true>(batch_pick(b.x, j), row, cols, batch_pick(b.ldx, j), margin, batch_pick(b.q, j),
                                 batch_pick(b.ldq, j), batch_pick(b.scale_inv, j), batch_pick(b.amax, j), b.nt_store);
}

// Rowwise casts with the per-column amax of each tensor as a side output (for
// a later colwise quantization of the same tensor: "FP8 Training on AMD GPUs
// with TorchTitan and TorchAO", colwise scales), in the same single pass over
// x. Tensor j owns workgroups first[j] .. first[j+1]-1 (about one per CU in
// all), which stride over its rows, a wavefront per row at a time. The
// workgroup's column maxima meet in LDS as fp32 bit patterns (relaxed LDS max)
// at index (col % 8) * 64 MAXC + col / 8, so the 64 lanes of one LDS max touch
// 64 consecutive words. REG: each wavefront keeps the running packed magnitude
// max of its chunks in registers and folds it into LDS once at the end (rows
// of up to 8 chunks per lane); otherwise it folds every row into LDS right
// after casting it (longer rows leave no registers for a running max). PREF:
// each wavefront loads its next row before casting the current one (two rows
// in registers). At the end
// each column is folded into col_amax[j] (cleared beforehand) by one relaxed
// atomic max per workgroup, skipped where the workgroup saw only zeros: with
// one workgroup per CU the atomics stay few (one per column per CU).
// Grouped column amax (ngroups[j] = G > 0: the per-group column amax that a
// later grouped colwise cast of the same tensor takes as ready, e.g. MoE
// tokens sorted by expert): each workgroup takes a contiguous band of rows
// instead, cut where a group ends; after each piece its maxima go to
// col_amax[j][g * cols + c] of that piece's group g and LDS is cleared for the
// next. Rows of no group (before offsets[0] or past offsets[G]) are cast but
// fold nowhere.
template <int MAXC>
__device__ __forceinline__ void load_row_chunks(uint4 (&v)[MAXC], const uint16_t* __restrict__ x, int64_t row,
                                                int64_t ldx, int nch) {
    const int lane = threadIdx.x & 63;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));   // past the row: a duplicate chunk, never used
    }
}

template <int F, int MAXC>
__device__ __forceinline__ void cast_row_chunks(const uint4 (&v)[MAXC], int64_t row, int nch, int margin,
                                                uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale_inv,
                                                float* __restrict__ amax_out, int nt_store) {
    const int lane = threadIdx.x & 63;
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
            if (ch >= nch) continue;
            const uint2 code = encode8<F, true>(v[c], s);
            if (nt_store)
                __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, code),
                                            reinterpret_cast<unsigned long long*>(&qr[ch]));
            else
                qr[ch] = code;
        }
    } else {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            if (ch < nch) qr[ch] = encode8<F, false>(v[c], s);
        }
    }
}

// Folds packed magnitude words (chunk layout) into the LDS column maxima:
// column col at word (col % 8) * MAXC * 64 + col / 8 (so every address is the
// lane's word plus a compile-time offset).
template <int MAXC>
__device__ __forceinline__ void fold_chunks_lds(const uint4 (&w)[MAXC], uint32_t* red, int nch) {
    constexpr int kSeg = MAXC * 64;
    const int lane = threadIdx.x & 63;
    uint32_t* base = red + lane;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        if (lane + c * 64 >= nch) continue;
        const uint32_t a[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            __hip_atomic_fetch_max(base + (2 * k) * kSeg + c * 64, (a[k] & 0xffffu) << 16, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_max(base + (2 * k + 1) * kSeg + c * 64, a[k] & 0xffff0000u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
}

template <int F, int MAXC, int WAVES, bool REG, bool PREF, bool GROUPED>
__global__ __launch_bounds__(WAVES * 64) void k_quant_row_colmax(RowBatch b, int64_t cols, int margin) {
    constexpr int kCols = MAXC * 64 * 8;                 // columns a row of MAXC chunks per lane can hold
    __shared__ uint32_t red[kCols];
    const int64_t bid = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i < b.count && bid >= b.first[i]) j = i;
    int64_t first = b.first[0], next = b.first[1];
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i == j) {
            first = b.first[i];
            next = b.first[i + 1];
        }
    const int wave = threadIdx.x >> 6;
    const int nch = (int)(cols >> 3);
    const int64_t rows = batch_pick(b.rows, j);
    float* cam = batch_pick(b.col_amax, j);
    for (int i = threadIdx.x; i < kCols; i += WAVES * 64) red[i] = 0u;
    __syncthreads();
    const uint16_t* x = batch_pick(b.x, j);
    uint8_t* q = batch_pick(b.q, j);
    float* si = batch_pick(b.scale_inv, j);
    float* am = batch_pick(b.amax, j);
    const int64_t ldx = batch_pick(b.ldx, j), ldq = batch_pick(b.ldq, j);
    const int64_t stride = (next - first) * WAVES;
    uint4 cm[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) cm[c] = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (GROUPED) {
        // every tensor of the batch by bands; an ungrouped column amax is one
        // group of all rows, a tensor without column amax has no group
        const int64_t* off = batch_pick(b.groups, j);
        const int G = cam ? (batch_pick(b.ngroups, j) > 0 ? batch_pick(b.ngroups, j) : 1) : 0;
        auto start = [&](int g) {                        // offsets[g] clamped to [0, rows]
            if (off == nullptr) return g == 0 && G > 0 ? (int64_t)0 : rows;
            const int64_t v = off[g];
            return v < 0 ? 0 : (v > rows ? rows : v);
        };
        const int64_t band = (rows + (next - first) - 1) / (next - first);
        const int64_t lo = (bid - first) * band;
        const int64_t hi = lo + band < rows ? lo + band : rows;
        for (int64_t s = lo; s < hi;) {
            // the piece [s, e): rows of group g (the last whose start is <= s)
            // up to its end, or rows of no group (g = -1) up to the next start
            int glo = -1, ghi = G;
            while (ghi - glo > 1) {
                const int mid = (glo + ghi) >> 1;
                if (start(mid) <= s)
                    glo = mid;
                else
                    ghi = mid;
            }
            int g = glo;
            int64_t e;
            if (g >= 0 && start(g + 1) > s) {
                e = start(g + 1) < hi ? start(g + 1) : hi;
            } else {
                const int64_t nx = start(g + 1);
                e = nx > s && nx < hi ? nx : hi;
                g = -1;
            }
            for (int64_t r = s + wave; r < e; r += WAVES) {
                uint4 cur[MAXC];
                load_row_chunks<MAXC>(cur, x, r, ldx, nch);
                cast_row_chunks<F, MAXC>(cur, r, nch, margin, q, ldq, si, am, b.nt_store);
#pragma unroll
                for (int c = 0; c < MAXC; ++c) {
                    cur[c].x &= 0x7fff7fffu;
                    cur[c].y &= 0x7fff7fffu;
                    cur[c].z &= 0x7fff7fffu;
                    cur[c].w &= 0x7fff7fffu;
                }
                if constexpr (REG) {
#pragma unroll
                    for (int c = 0; c < MAXC; ++c) {
                        cm[c].x = pk_absmax(cm[c].x, cur[c].x);
                        cm[c].y = pk_absmax(cm[c].y, cur[c].y);
                        cm[c].z = pk_absmax(cm[c].z, cur[c].z);
                        cm[c].w = pk_absmax(cm[c].w, cur[c].w);
                    }
                } else if (g >= 0) {
                    fold_chunks_lds<MAXC>(cur, red, nch);
                }
            }
            if (g >= 0) {                                // (uniform)
                if constexpr (REG) fold_chunks_lds<MAXC>(cm, red, nch);
                __syncthreads();
                float* cg = cam + (int64_t)g * cols;
                for (int i = threadIdx.x; i < cols; i += WAVES * 64) {
                    const int k = (i & 7) * (MAXC * 64) + (i >> 3);
                    const uint32_t v32 = red[k];
                    if (v32 != 0u) {
                        atomic_max_bits(cg + i, v32);
                        red[k] = 0u;
                    }
                }
                __syncthreads();                         // LDS clear before the next piece folds
            }
#pragma unroll
            for (int c = 0; c < MAXC; ++c) cm[c] = make_uint4(0u, 0u, 0u, 0u);
            s = e;
        }
        return;
    }
    int64_t row = (bid - first) * WAVES + wave;
    uint4 v[MAXC];
    if (PREF && row < rows) load_row_chunks<MAXC>(v, x, row, ldx, nch);
    while (row < rows) {
        uint4 cur[MAXC];
        const int64_t nrow = row + stride;
        if constexpr (PREF) {
#pragma unroll
            for (int c = 0; c < MAXC; ++c) cur[c] = v[c];
            if (nrow < rows) load_row_chunks<MAXC>(v, x, nrow, ldx, nch);     // the next row is in flight meanwhile
        } else {
            load_row_chunks<MAXC>(cur, x, row, ldx, nch);
        }
        cast_row_chunks<F, MAXC>(cur, row, nch, margin, q, ldq, si, am, b.nt_store);
        if (cam) {
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                cur[c].x &= 0x7fff7fffu;
                cur[c].y &= 0x7fff7fffu;
                cur[c].z &= 0x7fff7fffu;
                cur[c].w &= 0x7fff7fffu;
            }
            if constexpr (REG) {
#pragma unroll
                for (int c = 0; c < MAXC; ++c) {
                    cm[c].x = pk_absmax(cm[c].x, cur[c].x);
                    cm[c].y = pk_absmax(cm[c].y, cur[c].y);
                    cm[c].z = pk_absmax(cm[c].z, cur[c].z);
                    cm[c].w = pk_absmax(cm[c].w, cur[c].w);
                }
            } else {
                fold_chunks_lds<MAXC>(cur, red, nch);
            }
        }
        row = nrow;
    }
    if (cam == nullptr) return;                          // (uniform over the workgroup)
    if constexpr (REG) fold_chunks_lds<MAXC>(cm, red, nch);
    __syncthreads();
    for (int i = threadIdx.x; i < cols; i += WAVES * 64) {
        const uint32_t v32 = red[(i & 7) * (MAXC * 64) + (i >> 3)];
        if (v32 != 0u) atomic_max_bits(cam + i, v32);
    }
}

// Clears the column-amax outputs of a batch in one launch (tensor j's
// cam_first[j + 1] - cam_first[j] floats: cols, or G * cols when grouped).
__global__ void k_fill_col_amax(RowBatch b) {
    const int64_t n = b.cam_first[b.count];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        int j = 0;
#pragma unroll
        for (int t = 1; t < kMaxRowBatch; ++t)
            if (t < b.count && i >= b.cam_first[t]) j = t;
        float* cam = batch_pick(b.col_amax, j);
        int64_t f = b.cam_first[0];
#pragma unroll
        for (int t = 1; t < kMaxRowBatch; ++t)
            if (t == j) f = b.cam_first[t];
        if (cam) cam[i - f] = 0.0f;
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

// Tensorwise cast with the row in registers (one wavefront per row, MAXC
// 16-byte chunks per lane). DELAYED: the scale comes from the state and the
// tensor's amax is folded into amax_io (the row's own amax picks the encoder:
// a row holding a NaN takes the bit-level one); otherwise the scale comes from
// amax_io, which the amax pass filled, and a NaN amax sends every row to the
// bit-level encoder.
// The rows of one tensor taken by workgroup `wg` of the `nwg` that share it
// (red: kWaves words of LDS for the workgroup's amax).
template <int F, int MAXC, bool DELAYED>
__device__ __forceinline__ void quant_tensor_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  int64_t ldx, int margin, const float* __restrict__ scale,
                                                  uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale_inv,
                                                  float* __restrict__ amax_io, int64_t wg, int64_t nwg,
                                                  uint32_t* red) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = nwg * kWaves;
    const float s = DELAYED ? *scale : scale_from_amax<F>(*amax_io, margin);
    const bool tensor_nan = DELAYED ? false : __builtin_isnan(*amax_io);
    if (wg == 0 && threadIdx.x == 0) scale_inv[0] = 1.0f / s;
    const int nch = (int)(cols >> 3);
    uint32_t mx = 0;
    for (int64_t row = wg * kWaves + (threadIdx.x >> 6); row < rows; row += nwaves) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
        uint4 v[MAXC];
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));     // past the row: a duplicate chunk, never stored
        }
        bool nan_row = tensor_nan;
        if (DELAYED) {
            uint32_t rm = 0;
#pragma unroll
            for (int c = 0; c < MAXC; ++c) rm = word_absmax(rm, v[c]);
            rm = pk_fold(rm);
            mx = rm > mx ? rm : mx;
            nan_row = nan_bits16(wave_max_u32(rm));
        }
        uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
        if (!nan_row) {
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                const int ch = lane + c * 64;
                if (ch < nch) qr[ch] = encode8<F, true>(v[c], s);
            }
        } else {
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                const int ch = lane + c * 64;
                if (ch < nch) qr[ch] = encode8<F, false>(v[c], s);
            }
        }
    }
    if (DELAYED) {
        mx = block_max_u32(mx, red);
        if (threadIdx.x == 0) atomic_max_bits(amax_io, mx << 16);
    }
}

template <int F, int MAXC, bool DELAYED>
__global__ __launch_bounds__(kBlock) void k_quant_tensor_reg(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx, int margin,
                                                             const float* __restrict__ scale, uint8_t* __restrict__ q,
                                                             int64_t ldq, float* __restrict__ scale_inv,
                                                             float* __restrict__ amax_io) {
    __shared__ uint32_t red[kWaves];
    quant_tensor_rows<F, MAXC, DELAYED>(x, rows, cols, ldx, margin, scale, q, ldq, scale_inv, amax_io, blockIdx.x,
                                        gridDim.x, red);
}

// Delayed tensorwise casts of up to kMaxRowBatch tensors with the same number
// of columns in one launch (a linear layer's X and W, each with its own
// delayed scale and amax): tensor j owns workgroups first[j] .. first[j+1]-1
// (at least one), which stride over its rows as above.
struct TensorBatch {
    const uint16_t* x[kMaxRowBatch];
    uint8_t* q[kMaxRowBatch];
    const float* scale[kMaxRowBatch];
    float* scale_inv[kMaxRowBatch];
    float* amax[kMaxRowBatch];
    int64_t rows[kMaxRowBatch];
    int64_t ldx[kMaxRowBatch];
    int64_t ldq[kMaxRowBatch];
    int64_t first[kMaxRowBatch + 1];
    int count;
};

template <int F, int MAXC>
__global__ __launch_bounds__(kBlock) void k_quant_tensor_batch(TensorBatch b, int64_t cols) {
    __shared__ uint32_t red[kWaves];
    const int64_t bid = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i < b.count && bid >= b.first[i]) j = i;
    int64_t first = b.first[0], next = b.first[1];
#pragma unroll
    for (int i = 1; i < kMaxRowBatch; ++i)
        if (i == j) {
            first = b.first[i];
            next = b.first[i + 1];
        }
    const int64_t nwg = next - first;
    quant_tensor_rows<F, MAXC, true>(batch_pick(b.x, j), batch_pick(b.rows, j), cols, batch_pick(b.ldx, j), 0,
                                     batch_pick(b.scale, j), batch_pick(b.q, j), batch_pick(b.ldq, j),
                                     batch_pick(b.scale_inv, j), batch_pick(b.amax, j), bid - first, nwg, red);
}

// --------------------------------------------------------------- MX quantizer --
// MXFP8 rowwise: blocks of 32 consecutive elements of a row share a
// power-of-two scale 2^e stored as e + 127 (E8M0; 0xFF for a block holding a
// NaN or Inf, whose elements are then cast with scale 1), e = floor(log2 amax)
// - emax (8 for e4m3, 15 for e5m2) clamped to [-127, 127], e = -127 for a zero
// block; elements are the saturating RNE cast of x * 2^-e (a reading of the
// MXFP8 the TorchTitan/TorchAO page names; the pages define no format). One
// wavefront per row slice of up to kMxSlice columns (grid y), held in
// registers; a block is 4 lanes' 16-byte chunks, reduced with two lane
// exchanges. Scale layout, K-step major: the scales of blocks 4j .. 4j+3 of
// row r are the 4 bytes at sc + 4 (j ldsc + r) (so the rows of one 128-deep K
// step are contiguous for the GEMM); the lane holding the first chunk of
// blocks 4j .. 4j+3 gathers their bytes and stores the dword, with zero bytes
// for blocks past the row.
template <int F>
__device__ __forceinline__ constexpr int mx_emax() { return F == kE4M3 ? 8 : 15; }

constexpr int64_t kMxSlice = 32 * 64 * 8;               // 16384 columns: 32 chunks per lane

// The scale records of a workgroup's W rows are gathered in LDS and stored one
// K step at a time (the step's W records are contiguous in the K-step-major
// layout): one W * 4-byte store per step instead of W scattered 4-byte stores.
constexpr int kRecSteps = (int)(kMxSlice / 128);       // records per row of one slice

template <int W>
__device__ __forceinline__ void store_records(const uint32_t* rec, int nrec, uint8_t* __restrict__ sc, int64_t ldsc,
                                              int64_t row0, int64_t rows) {
    __syncthreads();
    for (int i = threadIdx.x; i < nrec * W; i += W * 64) {
        const int j = i / W, r = i % W;
        if (row0 + r < rows) *reinterpret_cast<uint32_t*>(sc + 4 * ((int64_t)j * ldsc + row0 + r)) = rec[i];
    }
}

template <int F, int MAXC, int W>
__global__ __launch_bounds__(W * 64) void k_mx_quant_row(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                                                         uint8_t* __restrict__ sc, int64_t ldsc) {
    __shared__ uint32_t rec[kRecSteps * W];
    const int lane = threadIdx.x & 63;
    const int rl = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * W;
    const int64_t row = row0 + rl;
    const int64_t c0 = (int64_t)blockIdx.y * kMxSlice;
    x += c0;
    q += c0;
    sc += (c0 / 128) * ldsc * 4;
    const int nch = (int)((cols - c0 < kMxSlice ? cols - c0 : kMxSlice) >> 3);
    if (row < rows) {                                    // (uniform over the wavefront)
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));     // past the row: a duplicate chunk, never stored
    }
    uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        uint32_t mx = pk_fold(word_absmax(0u, v[c]));
        uint32_t o = __shfl_xor(mx, 1);
        mx = o > mx ? o : mx;
        o = __shfl_xor(mx, 2);
        mx = o > mx ? o : mx;                            // the block's amax (16-bit magnitude bits)
        uint32_t e8;
        float mul;
        if (mx >= 0x7f80u) {                             // Inf or NaN in the block
            e8 = 0xFFu;
            mul = 1.0f;
        } else if (mx == 0u) {
            e8 = 0u;
            mul = 1.0f;                                  // (zeros cast to zero at any scale)
        } else {
            // floor(log2 amax) from the bf16 magnitude bits: the exponent field,
            // or for a subnormal (field 0) the position of the top mantissa bit
            const int fld = (int)(mx >> 7);
            const int lg = fld > 0 ? fld - 127 : (31 - __builtin_clz(mx)) - 133;
            int e = lg - mx_emax<F>();
            e = e < -127 ? -127 : (e > 127 ? 127 : e);
            e8 = (uint32_t)(e + 127);
            mul = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal float for every e reachable here
        }
        if (ch < nch) qr[ch] = e8 != 0xFFu ? encode8<F, true>(v[c], mul) : encode8<F, false>(v[c], mul);
        // lanes 16i, 16i+4, 16i+8, 16i+12 hold the first chunks of blocks 4j .. 4j+3
        const uint32_t mine = ch < nch ? e8 : 0u;
        const uint32_t b1 = __shfl_down(mine, 4), b2 = __shfl_down(mine, 8), b3 = __shfl_down(mine, 12);
        if ((lane & 15) == 0 && ch < nch) rec[(ch >> 4) * W + rl] = mine | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    }
    store_records<W>(rec, (nch + 15) / 16, sc, ldsc, row0, rows);
}

// ---------------------------------------------------------- blockwise casts --
// Blockwise recipe: 1 x 128 blocks along K for activations, 128 x 128 tiles for
// weights, one scale per block: the current-scaling scale fmax / amax (1 for a
// zero or non-finite amax, FLT_MAX at most) rounded down to a power of two (its
// mantissa bits cleared), so no element saturates (a reading of the blockwise
// recipe the Flux page lists; the pages give no shapes or rule). The scale is
// stored as the E8M0 byte of 1 / s, 254 - (exponent field of s), in the K-step
// major records of the MX entry points (all four bytes of a record equal: a
// 128-deep K step is one block), so the products run as MX products.
__device__ __forceinline__ float pow2_floor(float s) { return __uint_as_float(__float_as_uint(s) & 0xff800000u); }
__device__ __forceinline__ uint32_t e8m0_of_inverse(float s_pow2) { return 254u - (__float_as_uint(s_pow2) >> 23); }

// One wavefront per row slice of up to kMxSlice columns (grid y), in registers;
// a 128-block is 16 lanes' chunks, reduced with four lane exchanges; the lane
// holding a block's first chunk stores its record.
template <int F, int MAXC, int W>
__global__ __launch_bounds__(W * 64) void k_blockwise_quant_act(const uint16_t* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ldx, uint8_t* __restrict__ q,
                                                                int64_t ldq, uint8_t* __restrict__ sc,
                                                                int64_t ldsc) {
    __shared__ uint32_t rec[kRecSteps * W];
    const int lane = threadIdx.x & 63;
    const int rl = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * W;
    const int64_t row = row0 + rl;
    const int64_t c0 = (int64_t)blockIdx.y * kMxSlice;
    x += c0;
    q += c0;
    sc += (c0 / 128) * ldsc * 4;
    const int nch = (int)((cols - c0 < kMxSlice ? cols - c0 : kMxSlice) >> 3);
    if (row < rows) {                                    // (uniform over the wavefront)
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));     // past the row: a duplicate chunk, never stored
    }
    uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        uint32_t mx = pk_fold(word_absmax(0u, v[c]));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const uint32_t y = __shfl_xor(mx, o);
            mx = y > mx ? y : mx;
        }
        const float amax = amax_from_bits16(mx);
        const float s = pow2_floor(scale_from_amax<F>(amax, 0));
        if (ch < nch) {
            qr[ch] = !__builtin_isnan(amax) ? encode8<F, true>(v[c], s) : encode8<F, false>(v[c], s);
            if ((lane & 15) == 0) rec[(ch >> 4) * W + rl] = e8m0_of_inverse(s) * 0x01010101u;
        }
    }
    }
    store_records<W>(rec, (nch + 15) / 16, sc, ldsc, row0, rows);
}

// One workgroup per 128 x 128 tile (kfast: grid x the K blocks and y the row
// tiles, so that consecutive workgroups read neighbouring 256-byte segments of
// the same rows, ~6% faster; otherwise x the row tiles and y the K blocks, for
// more than 65535 row tiles). Thread (wave w, lane l) holds chunk l % 16 of
// rows 16p + 4w + l / 16, p = 0..7 (rows past the matrix clamped to its last
// row); tile amax over the workgroup through LDS; threads holding chunk 0 store
// their rows' records.
template <int F>
__global__ __launch_bounds__(kBlock) void k_blockwise_quant_weight(const uint16_t* __restrict__ w, int64_t rows,
                                                                   int64_t ldw, uint8_t* __restrict__ q,
                                                                   int64_t ldq, uint8_t* __restrict__ sc,
                                                                   int64_t ldsc, int kfast) {
    __shared__ uint32_t red[kWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cc = lane & 15;
    const int64_t kb = kfast ? blockIdx.x : blockIdx.y;         // K block
    const int64_t r0 = (int64_t)(kfast ? blockIdx.y : blockIdx.x) * 128;
    const int64_t k0 = kb * 128;
    uint4 v[8];
    uint32_t mx = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = r0 + 16 * p + 4 * wave + (lane >> 4);
        const int64_t rc = r < rows ? r : rows - 1;
        v[p] = load_stream(reinterpret_cast<const uint4*>(w + rc * ldw + k0 + 8 * cc));
        mx = word_absmax(mx, v[p]);
    }
    mx = wave_max_u32(pk_fold(mx));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) mx = red[i] > mx ? red[i] : mx;
    const float amax = amax_from_bits16(mx);
    const float s = pow2_floor(scale_from_amax<F>(amax, 0));
    const uint32_t rec = e8m0_of_inverse(s) * 0x01010101u;
    const bool nan_free = !__builtin_isnan(amax);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = r0 + 16 * p + 4 * wave + (lane >> 4);
        if (r >= rows) continue;
        *reinterpret_cast<uint2*>(q + r * ldq + k0 + 8 * cc) = nan_free ? encode8<F, true>(v[p], s)
                                                                        : encode8<F, false>(v[p], s);
        if (cc == 0) *reinterpret_cast<uint32_t*>(sc + 4 * (kb * ldsc + r)) = rec;
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
        if (scale_inv && c < cols) scale_inv[c] = 1.0f / s;
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

// Loads of one 128 x 64 tile: source rows r0 .. r0+127 (rows at or past
// src_end read as row src_end-1, or as zeros when zero_past_end), columns
// c0 .. c0+63; thread (cc = t % 8, rg = t / 8) takes rows 4rg .. 4rg+3 of
// columns 8cc .. 8cc+7. Rows / columns past the end re-read the last row /
// chunk, so the loads stay unconditional (all four in flight together); those
// codes are never stored, or become zeros when zero_past_end.
__device__ __forceinline__ void col_tile_load(uint4 (&v)[4], const uint16_t* __restrict__ x, int64_t ldx, int64_t r0,
                                              int64_t src_end, bool zero_past_end, int64_t c0, int64_t cols) {
    const int t = threadIdx.x;
    const int cc = t & 7, rg = t >> 3;
    const int64_t col = c0 + cc * 8;
    const int64_t lcol = col < cols ? col : cols - 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + rg * 4 + r;
        v[r] = *reinterpret_cast<const uint4*>(x + (row < src_end ? row : src_end - 1) * ldx + lcol);
        if (zero_past_end && row >= src_end) v[r] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Casts the loaded rows with the column scales s_lds / nan_lds and writes them
// transposed into the LDS tile (no barrier).
template <int F>
__device__ __forceinline__ void col_tile_encode(const uint4 (&v)[4], const float* s_lds, const int* nan_lds,
                                               uint32_t* tile) {
    const int t = threadIdx.x;
    const int cc = t & 7, rg = t >> 3;
    uint32_t w[4][2];
    float s[8];
    int any_nan = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s[j] = s_lds[cc * 8 + j];
        any_nan |= nan_lds[cc * 8 + j];
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
}

// Writes the LDS tile transposed to qt rows c0 .. (one per column) at columns
// d0 .. d0+127, none at or past d_end (after a barrier).
__device__ __forceinline__ void col_tile_store(const uint32_t* tile, int64_t c0, int64_t cols,
                                               uint8_t* __restrict__ qt, int64_t ldqt, int64_t d0, int64_t d_end,
                                               int vec_store) {
    const int t = threadIdx.x;
    // 64 columns x 8 chunks of 16 bytes; two per thread
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = t + i * kBlock;
        const int lc = p >> 3, rc = p & 7;
        const int64_t ocol = c0 + lc;
        if (ocol >= cols) continue;
        const int sw = (rc ^ (lc >> 3)) & 7;
        const uint4 val = *reinterpret_cast<const uint4*>(&tile[lc * (kColTileR / 4) + sw * 4]);
        const int64_t orow = d0 + rc * 16;
        uint8_t* dst = qt + ocol * ldqt + orow;
        if (vec_store && orow + 16 <= d_end) {
            *reinterpret_cast<uint4*>(dst) = val;
        } else {
            const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
            for (int b = 0; b < 16 && orow + b < d_end; ++b) dst[b] = (uint8_t)(wv[b >> 2] >> (8 * (b & 3)));
        }
    }
}

// One 128 x 64 tile (load, cast, transpose through LDS, store): source rows
// r0 .. r0+127 of columns c0 .. c0+63 to qt rows c0 .. at columns d0 ...
template <int F>
__device__ __forceinline__ void col_tile(const uint16_t* __restrict__ x, int64_t ldx, int64_t r0, int64_t src_end,
                                         bool zero_past_end, int64_t c0, int64_t cols, const float* s_lds,
                                         const int* nan_lds, uint32_t* tile, uint8_t* __restrict__ qt, int64_t ldqt,
                                         int64_t d0, int64_t d_end, int vec_store) {
    uint4 v[4];
    col_tile_load(v, x, ldx, r0, src_end, zero_past_end, c0, cols);
    col_tile_encode<F>(v, s_lds, nan_lds, tile);
    __syncthreads();
    col_tile_store(tile, c0, cols, qt, ldqt, d0, d_end, vec_store);
}

// The colwise cast's workgroup takes kColTilesPerWg tiles side by side (128
// rows x 256 columns): its loads of one row are a 512-byte run, and all 16 of a
// thread's loads are issued before the first is cast. The grid's x runs over
// the column blocks, so workgroups dispatched together read neighbouring runs
// of the same rows; y (plus y_base, for grids over 65535 row tiles) over the
// row tiles. The row tile 0 workgroups write scale_inv.
constexpr int kColTilesPerWg = 4;

template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_col_tiled(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, int margin,
                                                            uint8_t* __restrict__ qt, int64_t ldqt,
                                                            float* __restrict__ scale_inv,
                                                            const float* __restrict__ col_amax, int vec_store,
                                                            int64_t y_base) {
    constexpr int SC = kColTilesPerWg;
    __shared__ float s_lds[kColTileC * SC];
    __shared__ int nan_lds[kColTileC * SC];
    __shared__ __attribute__((aligned(16))) uint32_t tile[SC][kColTileC * kColTileR / 4];
    const int64_t c0 = (int64_t)blockIdx.x * kColTileC * SC;
    const int64_t ty = y_base + blockIdx.y;
    const int64_t r0 = ty * kColTileR;
    if (threadIdx.x < kColTileC * SC) {
        const int64_t c = c0 + threadIdx.x;
        const float a = c < cols ? col_amax[c] : 0.0f;
        const float sc = scale_from_amax<F>(a, margin);
        s_lds[threadIdx.x] = sc;
        nan_lds[threadIdx.x] = __builtin_isnan(a) ? 1 : 0;
        if (ty == 0 && c < cols) scale_inv[c] = 1.0f / sc;
    }
    uint4 v[SC][4];
#pragma unroll
    for (int j = 0; j < SC; ++j) col_tile_load(v[j], x, ldx, r0, rows, false, c0 + kColTileC * j, cols);
    __syncthreads();                                     // the column scales are in LDS
#pragma unroll
    for (int j = 0; j < SC; ++j) col_tile_encode<F>(v[j], s_lds + kColTileC * j, nan_lds + kColTileC * j, tile[j]);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SC; ++j) col_tile_store(tile[j], c0 + kColTileC * j, cols, qt, ldqt, r0, rows, vec_store);
}

// Dual cast of one tensor (rowwise codes and colwise-transposed codes, e.g.
// the gradient dY of a linear layer, which its dgrad takes rowwise and its
// wgrad colwise: "FP8 training for Flux models", fp8 hybrid and fp8_wgrad;
// "FP8 Training on AMD GPUs with TorchTitan and TorchAO", colwise scales),
// second pass: with the row and column amax known, each 128 x 64 tile is read
// once and cast twice. Row codes, with the scales of the tile's 128 rows (in
// LDS), go straight out in x's layout (8 lanes per 64-byte row segment);
// column codes go through the LDS transpose as in k_quant_col_tiled.
template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_rowcol_tiled(const uint16_t* __restrict__ x, int64_t rows,
                                                               int64_t cols, int64_t ldx, int margin,
                                                               uint8_t* __restrict__ q, int64_t ldq,
                                                               float* __restrict__ row_scale_inv,
                                                               const float* __restrict__ row_amax,
                                                               uint8_t* __restrict__ qt, int64_t ldqt,
                                                               float* __restrict__ col_scale_inv,
                                                               const float* __restrict__ col_amax, int vec_store) {
    __shared__ float s_lds[kColTileC];
    __shared__ int nan_lds[kColTileC];
    __shared__ float rs_lds[kColTileR];
    __shared__ int rnan_lds[kColTileR];
    __shared__ __attribute__((aligned(16))) uint32_t tile[kColTileC * kColTileR / 4];
    const int64_t c0 = (int64_t)blockIdx.y * kColTileC;
    const int64_t r0 = (int64_t)blockIdx.x * kColTileR;
    const int t = threadIdx.x;
    if (t < kColTileR) {
        const int64_t r = r0 + t;
        const float a = r < rows ? row_amax[r] : 0.0f;
        const float sr = scale_from_amax<F>(a, margin);
        rs_lds[t] = sr;
        rnan_lds[t] = __builtin_isnan(a) ? 1 : 0;
        if (blockIdx.y == 0 && r < rows) row_scale_inv[r] = 1.0f / sr;
    }
    col_scales_to_lds<F>(col_amax, c0, cols, margin, blockIdx.x == 0 ? col_scale_inv : nullptr, s_lds, nan_lds);
    uint4 v[4];
    col_tile_load(v, x, ldx, r0, rows, false, c0, cols);
    const int cc = t & 7, rg = t >> 3;
    const int64_t col = c0 + cc * 8;
    if (col < cols) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int lr = rg * 4 + r;
            const int64_t row = r0 + lr;
            if (row >= rows) continue;
            const uint2 code = rnan_lds[lr] ? encode8<F, false>(v[r], rs_lds[lr]) : encode8<F, true>(v[r], rs_lds[lr]);
            *reinterpret_cast<uint2*>(q + row * ldq + col) = code;
        }
    }
    col_tile_encode<F>(v, s_lds, nan_lds, tile);
    __syncthreads();
    col_tile_store(tile, c0, cols, qt, ldqt, r0, rows, vec_store);
}

// ------------------------------------------------- grouped colwise (MoE) --

// Groups of at most kSmallGroupRows rows take the one-pass kernel
// (k_grouped_quant_col_small, 32-column strips); larger ones the two passes.
constexpr int kSmallGroupRows = 2048;
constexpr int kSmallStrip = 32;

// Row range of group g: offsets clamped to [0, total], hi >= lo.
__device__ __forceinline__ void group_rows(const int64_t* __restrict__ off, int g, int64_t total, int64_t* lo,
                                           int64_t* hi) {
    int64_t a = off[g], b = off[g + 1];
    a = a < 0 ? 0 : (a > total ? total : a);
    b = b < a ? a : (b > total ? total : b);
    *lo = a;
    *hi = b;
}

// Per-group column amax. A workgroup covers 512 columns of a band of 256 rows
// and walks the groups that meet the band (the first by binary search over the
// offsets): for each, the rows of the band inside the group are reduced as in
// k_amax_cols_vec and folded by one atomic per column into out[g * cols + c]
// (cleared beforehand).
__global__ __launch_bounds__(kBlock) void k_grouped_amax_cols(const uint16_t* __restrict__ x, int64_t total,
                                                              int64_t cols, int64_t ldx,
                                                              const int64_t* __restrict__ off, int G,
                                                              float* __restrict__ out, int skip_small) {
    __shared__ uint32_t part[kWaves][256];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ch = (int64_t)blockIdx.y * 64 + lane;
    const int64_t nch = cols >> 3;
    int64_t r0 = (int64_t)blockIdx.x * kColAmaxRows;
    const int64_t r1 = r0 + kColAmaxRows < total ? r0 + kColAmaxRows : total;
    // first group whose rows reach past r0: the last g with a clamped start <= r0
    int glo = 0, ghi = G;
    while (ghi - glo > 1) {
        const int mid = (glo + ghi) >> 1;
        int64_t a = off[mid];
        a = a < 0 ? 0 : (a > total ? total : a);
        if (a <= r0)
            glo = mid;
        else
            ghi = mid;
    }
    for (int g = glo; g < G && r0 < r1; ++g) {
        int64_t lo, hi;
        group_rows(off, g, total, &lo, &hi);
        const int64_t a = r0 > lo ? r0 : lo, b = r1 < hi ? r1 : hi;
        if (b <= a) continue;                            // (uniform: the whole workgroup skips)
        if (skip_small && hi - lo <= kSmallGroupRows) {  // (done by the one-pass kernel)
            r0 = b;
            continue;
        }
        uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
        if (ch < nch) {
            const uint16_t* base = x + ch * 8;
            for (int64_t rb = a + wave; rb < b; rb += kColAmaxUnroll * kWaves) {
                uint4 v[kColAmaxUnroll];
#pragma unroll
                for (int u = 0; u < kColAmaxUnroll; ++u) {
                    const int64_t r = rb + u * kWaves;
                    v[u] = *reinterpret_cast<const uint4*>(base + (r < b ? r : b - 1) * ldx);   // duplicates are harmless
                }
#pragma unroll
                for (int u = 0; u < kColAmaxUnroll; ++u) {
                    m0 = pk_absmax(m0, v[u].x);
                    m1 = pk_absmax(m1, v[u].y);
                    m2 = pk_absmax(m2, v[u].z);
                    m3 = pk_absmax(m3, v[u].w);
                }
            }
        }
        part[wave][lane * 4 + 0] = m0;
        part[wave][lane * 4 + 1] = m1;
        part[wave][lane * 4 + 2] = m2;
        part[wave][lane * 4 + 3] = m3;
        __syncthreads();
        const int t = threadIdx.x;
        uint32_t w = part[0][t];
#pragma unroll
        for (int k = 1; k < kWaves; ++k) w = pk_absmax(w, part[k][t]);
        const int64_t col = (int64_t)blockIdx.y * 512 + 2 * t;
        float* og = out + (int64_t)g * cols;
        if (col < cols) atomic_max_bits(og + col, (w & 0xffffu) << 16);
        if (col + 1 < cols) atomic_max_bits(og + col + 1, w & 0xffff0000u);
        __syncthreads();                                 // part[] is reused by the next group
        r0 = b;
    }
}

// scale_inv[i] = 1 / s(amax[i]) for every group and column (empty groups: 1).
template <int F>
__global__ void k_scale_inv_from_amax(const float* __restrict__ amax, int64_t n, int margin,
                                      float* __restrict__ scale_inv) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        scale_inv[i] = 1.0f / scale_from_amax<F>(amax[i], margin);
}

// Grouped transposed cast. Group g is cut into rt_g = roundup(m_g, 256) / 128
// row tiles of 128; tile t of group g covers its rows t*128 .. t*128+127
// (zeros past m_g: the padding) and lands at qt columns P_g + t*128 .., where
// P_g = 128 * (rt_0 + .. + rt_{g-1}). Every workgroup forms those prefix sums
// in LDS once (256 threads, then a block scan), then strides over the row
// tiles (the grid's x extent is at most the host-side upper bound of the tile
// count, capped near eight workgroups per CU over the column tiles) and finds
// each tile's group by binary search. (One workgroup per tile slot spent ~20 us
// of the MoE backward's expert-weight cast, 32 x 2048 x 7168, on slots that
// only exit.)
constexpr int kMaxGroups = 4096;

template <int F>
__global__ __launch_bounds__(kBlock) void k_grouped_quant_col_tiled(const uint16_t* __restrict__ x, int64_t total,
                                                                    int64_t cols, int64_t ldx, int margin,
                                                                    const int64_t* __restrict__ off, int G,
                                                                    uint8_t* __restrict__ qt, int64_t ldqt,
                                                                    const float* __restrict__ col_amax,
                                                                    float* __restrict__ scale_inv, int vec_store,
                                                                    int skip_small) {
    __shared__ float s_lds[kColTileC];
    __shared__ int nan_lds[kColTileC];
    __shared__ __attribute__((aligned(16))) uint32_t tile[kColTileC * kColTileR / 4];
    __shared__ int32_t pre[kMaxGroups + 1];
    __shared__ int32_t wsum[kWaves];
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    auto row_tiles = [&](int g) {
        int64_t lo, hi;
        group_rows(off, g, total, &lo, &hi);
        return (int32_t)(2 * ((hi - lo + 255) / 256));
    };
    const int per = (G + kBlock - 1) / kBlock;
    const int e0 = t * per, e1 = e0 + per < G ? e0 + per : G;
    int32_t mine = 0;
    for (int e = e0; e < e1; ++e) mine += row_tiles(e);
    int32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int32_t run = incl - mine;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int e = e0; e < e1; ++e) {
        pre[e] = run;
        run += row_tiles(e);
    }
    if (t == kBlock - 1) pre[G] = run;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.y * kColTileC;
    // scale_inv of the empty groups (no row tile visits them), by the first
    // workgroup of each column tile; with skip_small the one-pass kernel wrote them
    if (blockIdx.x == 0 && !skip_small) {
        const int64_t c = c0 + (t & 63);
        for (int g = t >> 6; g < G; g += kWaves)
            if (pre[g + 1] == pre[g] && c < cols)
                scale_inv[(int64_t)g * cols + c] = 1.0f / scale_from_amax<F>(col_amax[(int64_t)g * cols + c], margin);
    }
    // row tiles y = blockIdx.x, blockIdx.x + gridDim.x, .. (uniform over the workgroup)
    for (int32_t y = (int32_t)blockIdx.x; y < pre[G]; y += (int32_t)gridDim.x) {
        int glo = 0, ghi = G;                            // pre[glo] <= y < pre[ghi]
        while (ghi - glo > 1) {
            const int mid = (glo + ghi) >> 1;
            if (pre[mid] <= y)
                glo = mid;
            else
                ghi = mid;
        }
        const int g = glo;
        const int64_t tt = y - pre[g];
        int64_t lo, hi;
        group_rows(off, g, total, &lo, &hi);
        if (skip_small && hi - lo <= kSmallGroupRows) continue;   // (done by the one-pass kernel)
        __syncthreads();                                 // the previous tile's LDS reads are done
        // (the group's first row tile also writes its scale_inv)
        col_scales_to_lds<F>(col_amax + (int64_t)g * cols, c0, cols, margin,
                             tt == 0 ? scale_inv + (int64_t)g * cols : nullptr, s_lds, nan_lds);
        const int64_t d0 = (int64_t)pre[g] * kColTileR + tt * kColTileR;
        col_tile<F>(x, ldx, lo + tt * kColTileR, hi, true, c0, cols, s_lds, nan_lds, tile, qt, ldqt, d0, ldqt,
                    vec_store);
    }
}

// Groups of at most kSmallGroupRows rows in one pass: a workgroup holds a
// group's whole 32-column strip in registers (thread t: chunk t % 4 of 8
// columns, rows 4 (t / 4 + 64 i) + j, i < 8, j < 4), reduces the column amax
// (lanes, then the four wavefronts through LDS), casts, transposes 4 x 4 byte
// blocks into an LDS tile [32 columns][2048 rows] and stores each column's
// padded range P_g .. P_g + roundup(m_g, 256) as 16-byte chunks (zero codes
// past m_g). It writes the group's column amax and scale_inv; workgroups of
// larger groups exit (the two-pass kernels take them). P_g is summed over the
// earlier groups by the workgroup's threads.
template <int F>
__global__ __launch_bounds__(kBlock) void k_grouped_quant_col_small(const uint16_t* __restrict__ x, int64_t total,
                                                                    int64_t cols, int64_t ldx, int margin,
                                                                    const int64_t* __restrict__ off, int G,
                                                                    uint8_t* __restrict__ qt, int64_t ldqt,
                                                                    float* __restrict__ scale_inv,
                                                                    float* __restrict__ col_amax) {
    __shared__ uint32_t tile[kSmallStrip][kSmallGroupRows / 4 + 1];   // (+1: rows of a column apart in banks)
    __shared__ uint32_t red[kWaves][4][4];
    __shared__ int64_t psum[kWaves];
    const int g = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t lo, hi;
    group_rows(off, g, total, &lo, &hi);
    const int64_t m = hi - lo;
    if (m > kSmallGroupRows) return;                     // uniform over the workgroup
    // P_g: the padded sizes of the earlier groups
    int64_t part = 0;
    for (int h = t; h < g; h += kBlock) {
        int64_t a, b;
        group_rows(off, h, total, &a, &b);
        part += (b - a + 255) / 256 * 256;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if (lane == 0) psum[wave] = part;
    const int cq = t & 3, rq = t >> 2;
    const int64_t c0 = (int64_t)blockIdx.y * kSmallStrip;
    const int64_t nch = cols >> 3;                       // chunks of 8 columns in a row
    const int64_t ch = c0 / 8 + cq;
    const int64_t chc = ch < nch ? ch : nch - 1;         // past the last column: a duplicate chunk, never stored
    const uint16_t* base = x + lo * ldx + chc * 8;
    uint4 v[8][4];
    const int64_t mlast = m > 0 ? m - 1 : 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = 4 * (rq + 64 * i) + j;
            v[i][j] = m > 0 ? load_stream(reinterpret_cast<const uint4*>(base + (r < m ? r : mlast) * ldx))
                            : make_uint4(0u, 0u, 0u, 0u);
        }
    uint32_t mx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {                    // (duplicated rows past m do not change a max)
            mx[0] = pk_absmax(mx[0], v[i][j].x);
            mx[1] = pk_absmax(mx[1], v[i][j].y);
            mx[2] = pk_absmax(mx[2], v[i][j].z);
            mx[3] = pk_absmax(mx[3], v[i][j].w);
        }
#pragma unroll
    for (int o = 4; o < 64; o <<= 1)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t y = __shfl_xor(mx[q], o);
            mx[q] = pk_absmax(mx[q], y & 0x7fff7fffu);
        }
    if (lane < 4)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][lane][q] = mx[q];
    __syncthreads();
    const int64_t P = psum[0] + psum[1] + psum[2] + psum[3];
    float s[8];
    bool nan_free = true;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t w = red[0][cq][q];
#pragma unroll
        for (int k = 1; k < kWaves; ++k) w = pk_absmax(w, red[k][cq][q]);
        const float a0 = amax_from_bits16(w & 0xffffu), a1 = amax_from_bits16(w >> 16);
        s[2 * q] = scale_from_amax<F>(a0, margin);
        s[2 * q + 1] = scale_from_amax<F>(a1, margin);
        nan_free = nan_free && !__builtin_isnan(a0) && !__builtin_isnan(a1);
        if (rq == 0 && ch < nch) {                       // the four threads of row group 0 publish
            const int64_t c = ch * 8 + 2 * q;
            col_amax[(int64_t)g * cols + c] = a0;
            col_amax[(int64_t)g * cols + c + 1] = a1;
            scale_inv[(int64_t)g * cols + c] = 1.0f / s[2 * q];
            scale_inv[(int64_t)g * cols + c + 1] = 1.0f / s[2 * q + 1];
        }
    }
    // cast (zero codes past m), 4 x 4 byte transposes, LDS tile [column][row word]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t w[4][2];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = 4 * (rq + 64 * i) + j;
            const uint4 u = r < m ? v[i][j] : make_uint4(0u, 0u, 0u, 0u);
            if (nan_free) {
                w[j][0] = encode4<F, true>(bf16_lo(u.x) * s[0], bf16_hi(u.x) * s[1], bf16_lo(u.y) * s[2],
                                           bf16_hi(u.y) * s[3]);
                w[j][1] = encode4<F, true>(bf16_lo(u.z) * s[4], bf16_hi(u.z) * s[5], bf16_lo(u.w) * s[6],
                                           bf16_hi(u.w) * s[7]);
            } else {
                w[j][0] = encode4<F, false>(bf16_lo(u.x) * s[0], bf16_hi(u.x) * s[1], bf16_lo(u.y) * s[2],
                                            bf16_hi(u.y) * s[3]);
                w[j][1] = encode4<F, false>(bf16_lo(u.z) * s[4], bf16_hi(u.z) * s[5], bf16_lo(u.w) * s[6],
                                            bf16_hi(u.w) * s[7]);
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t a_lo = __builtin_amdgcn_perm(w[1][h], w[0][h], 0x05010400u);
            const uint32_t a_hi = __builtin_amdgcn_perm(w[1][h], w[0][h], 0x07030602u);
            const uint32_t b_lo = __builtin_amdgcn_perm(w[3][h], w[2][h], 0x05010400u);
            const uint32_t b_hi = __builtin_amdgcn_perm(w[3][h], w[2][h], 0x07030602u);
            const uint32_t tcol[4] = {__builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u),
                                      __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u),
                                      __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u),
                                      __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u)};
#pragma unroll
            for (int c = 0; c < 4; ++c) tile[cq * 8 + h * 4 + c][rq + 64 * i] = tcol[c];
        }
    }
    __syncthreads();
    // each column's padded range: roundup(m, 256) bytes as 16-byte chunks
    const int64_t padded = (m + 255) / 256 * 256;
    const int nck = (int)(padded / 16);                  // chunks per column
    for (int p = t; p < kSmallStrip * nck; p += kBlock) {
        const int lc = p / nck, k = p - lc * nck;
        const int64_t col = c0 + lc;
        if (col >= cols || P + 16 * k >= ldqt) continue;    // (columns of qt at or past ldqt are never written)
        const uint32_t* src = &tile[lc][4 * k];
        const uint4 val = make_uint4(src[0], src[1], src[2], src[3]);
        *reinterpret_cast<uint4*>(qt + col * ldqt + P + 16 * k) = val;
    }
}

// Any layout: one thread per column of a band of rows (reads coalesce across
// threads, writes do not; this path is for layouts the tiled kernel rejects).
template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_col_scalar(const uint16_t* __restrict__ x, int64_t rows,
                                                             int64_t cols, int64_t ldx, int margin,
                                                             uint8_t* __restrict__ qt, int64_t ldqt,
                                                             float* __restrict__ scale_inv,
                                                             const float* __restrict__ col_amax, int transpose) {
    const int64_t col = (int64_t)blockIdx.y * kBlock + threadIdx.x;
    if (col >= cols) return;
    const float s = scale_from_amax<F>(col_amax[col], margin);
    if (blockIdx.x == 0) scale_inv[col] = 1.0f / s;
    const int64_t r0 = (int64_t)blockIdx.x * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    for (int64_t r = r0; r < r1; ++r)
        qt[transpose ? col * ldqt + r : r * ldqt + col] = (uint8_t)encode1<F>(bf16_lo(x[r * ldx + col]) * s);
}

// Colwise scales with the codes in x's own layout (q [rows x cols], no
// transpose): lane l of a workgroup takes columns 8l .. 8l+7 of its 512-column
// chunk (grid y), their scales formed once in registers, and wavefront w the
// rows w, w + 4, .. of its 256-row band (grid x): 16-byte loads, 8-byte stores.
template <int F>
__global__ __launch_bounds__(kBlock) void k_quant_col_rows(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                           int64_t ldx, int margin, uint8_t* __restrict__ q,
                                                           int64_t ldq, float* __restrict__ scale_inv,
                                                           const float* __restrict__ col_amax) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.y * 512 + lane * 8;
    if (c0 >= cols) return;                              // (cols % 8 == 0: a lane's chunk is whole or absent)
    float s[8];
    int any_nan = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float a = col_amax[c0 + j];
        s[j] = scale_from_amax<F>(a, margin);
        any_nan |= __builtin_isnan(a) ? 1 : 0;
        if (blockIdx.x == 0 && wave == 0) scale_inv[c0 + j] = 1.0f / s[j];
    }
    const int64_t r0 = (int64_t)blockIdx.x * kColRows;
    const int64_t r1 = r0 + kColRows < rows ? r0 + kColRows : rows;
    for (int64_t r = r0 + wave; r < r1; r += kWaves) {
        const uint4 v = *reinterpret_cast<const uint4*>(x + r * ldx + c0);
        uint2 o;
        if (!any_nan) {
            o.x = encode4<F, true>(bf16_lo(v.x) * s[0], bf16_hi(v.x) * s[1], bf16_lo(v.y) * s[2], bf16_hi(v.y) * s[3]);
            o.y = encode4<F, true>(bf16_lo(v.z) * s[4], bf16_hi(v.z) * s[5], bf16_lo(v.w) * s[6], bf16_hi(v.w) * s[7]);
        } else {
            o.x = encode4<F, false>(bf16_lo(v.x) * s[0], bf16_hi(v.x) * s[1], bf16_lo(v.y) * s[2], bf16_hi(v.y) * s[3]);
            o.y = encode4<F, false>(bf16_lo(v.z) * s[4], bf16_hi(v.z) * s[5], bf16_lo(v.w) * s[6], bf16_hi(v.w) * s[7]);
        }
        *reinterpret_cast<uint2*>(q + r * ldq + c0) = o;
    }
}

// ------------------------------------------------------ delayed scale update --

// One wavefront per tensor. The effective amax combines the value being
// recorded with the other L-1 ring slots (the slot at head is the one being
// overwritten), so no lane reads a slot another lane is writing.
__device__ __forceinline__ int ring_head(const int32_t* head, int L) {
    return ((*head % L) + L) % L;            // a corrupt head cannot index outside the ring
}

template <int F>
__device__ __forceinline__ void delayed_update_one(float* __restrict__ cur_amax, float* __restrict__ history, int h,
                                                   int64_t i, int L, int algo, int margin, float* __restrict__ scale,
                                                   float* __restrict__ scale_inv) {
    const int lane = threadIdx.x & 63;
    const float cur = cur_amax[i];
    float* hist = history + i * (int64_t)L;
    uint32_t mx = __float_as_uint(cur) & 0x7fffffffu;
    if (algo == 1) {
        // eight independent loads per lane in flight per pass over 512 slots
        for (int t0 = 0; t0 < L; t0 += 512) {
            uint32_t b[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * 64 + lane;
                b[u] = (t < L && t != h) ? (__float_as_uint(hist[t]) & 0x7fffffffu) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) mx = b[u] > mx ? b[u] : mx;
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

template <int F>
__global__ __launch_bounds__(kBlock) void k_delayed_update(float* __restrict__ cur_amax, float* __restrict__ history,
                                                           const int32_t* __restrict__ head, int64_t n, int L,
                                                           int algo, int margin, float* __restrict__ scale,
                                                           float* __restrict__ scale_inv) {
    const int64_t i = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (i >= n) return;
    delayed_update_one<F>(cur_amax, history, ring_head(head, L), i, L, algo, margin, scale, scale_inv);
}

__global__ void k_advance_head(int32_t* head, int L) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *head = (ring_head(head, L) + 1) % L;
}

// Few tensors: one workgroup updates all of them (wavefront w takes tensors
// w, w + 4, ..) and then advances the head, after a barrier, so every
// wavefront has read the old head first. One launch instead of two.
constexpr int64_t kDelayedFusedMax = 64;

template <int F>
__global__ __launch_bounds__(kBlock) void k_delayed_update_fused(float* __restrict__ cur_amax,
                                                                 float* __restrict__ history, int32_t* head,
                                                                 int64_t n, int L, int algo, int margin,
                                                                 float* __restrict__ scale,
                                                                 float* __restrict__ scale_inv) {
    const int h = ring_head(head, L);
    for (int64_t i = threadIdx.x >> 6; i < n; i += kWaves)
        delayed_update_one<F>(cur_amax, history, h, i, L, algo, margin, scale, scale_inv);
    __syncthreads();
    if (threadIdx.x == 0) *head = (h + 1) % L;
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
                         int64_t ldq, float* scale_inv, float* amax_out, bool reread, hipStream_t st) {
    const dim3 grid(grid_for_rows(rows)), block(kBlock);
    // (cols > 0: the register kernels read at least one chunk per row)
    const bool vec =
        cols > 0 && is_aligned(x, 16) && is_aligned(q, 8) && ldx % 8 == 0 && ldq % 8 == 0 && cols % 8 == 0;
    if (!vec) {
        hipLaunchKernelGGL((k_quant_row_2pass<F, false>), grid, block, 0, st, x, rows, cols, ldx, margin, q, ldq,
                           scale_inv, amax_out);
        return hipGetLastError();
    }
    const int64_t per_lane = (cols / 8 + 63) / 64;
    const int nts = streamed_codes(rows * cols);
#define FP8_ROW_CASE(C)                                                                                        \
    if (per_lane <= C) {                                                                                       \
        if (reread)                                                                                            \
            hipLaunchKernelGGL((k_quant_row_reg<F, C, false>), grid, block, 0, st, x, rows, cols, ldx, margin, \
                               q, ldq, scale_inv, amax_out, nts);                                              \
        else                                                                                                   \
            hipLaunchKernelGGL((k_quant_row_reg<F, C, true>), grid, block, 0, st, x, rows, cols, ldx, margin,  \
                               q, ldq, scale_inv, amax_out, nts);                                              \
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
hipError_t quant_col_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin, int transpose,
                         uint8_t* qt, int64_t ldqt, float* scale_inv, const float* col_amax, hipStream_t st) {
    const bool vec_in = is_aligned(x, 16) && ldx % 8 == 0 && cols % 8 == 0;
    if (!transpose) {
        if (vec_in && is_aligned(qt, 8) && ldqt % 8 == 0) {
            const dim3 grid((unsigned)((rows + kColRows - 1) / kColRows), (unsigned)((cols + 511) / 512));
            hipLaunchKernelGGL((k_quant_col_rows<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, qt, ldqt,
                               scale_inv, col_amax);
        } else {
            const dim3 grid((unsigned)((rows + kColRows - 1) / kColRows), (unsigned)((cols + kBlock - 1) / kBlock));
            hipLaunchKernelGGL((k_quant_col_scalar<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, qt,
                               ldqt, scale_inv, col_amax, 0);
        }
        return hipGetLastError();
    }
    if (vec_in) {
        const int vec_store = is_aligned(qt, 16) && ldqt % 16 == 0;
        const int64_t gx = (cols + kColTileC * kColTilesPerWg - 1) / (kColTileC * kColTilesPerWg);
        const int64_t ty = (rows + kColTileR - 1) / kColTileR;
        for (int64_t y0 = 0; y0 < ty; y0 += 65535) {     // the grid's y is at most 65535
            const int64_t gy = ty - y0 < 65535 ? ty - y0 : 65535;
            hipLaunchKernelGGL((k_quant_col_tiled<F>), dim3((unsigned)gx, (unsigned)gy), dim3(kBlock), 0, st, x, rows,
                               cols, ldx, margin, qt, ldqt, scale_inv, col_amax, vec_store, y0);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else {
        const dim3 grid((unsigned)((rows + kColRows - 1) / kColRows), (unsigned)((cols + kBlock - 1) / kBlock));
        hipLaunchKernelGGL((k_quant_col_scalar<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, qt, ldqt,
                           scale_inv, col_amax, 1);
    }
    return hipGetLastError();
}

// Chunks of 16 bytes per lane that hold a whole row of `cols` bf16 values in
// registers (1, 2, 4, .., 32), or 0 if the row is longer than that.
int reg_chunks(int64_t cols) {
    const int64_t per_lane = (cols / 8 + 63) / 64;
    for (int c = 1; c <= 32; c *= 2)
        if (per_lane <= c) return c;
    return 0;
}

// Workgroups for the grid-stride tensor kernels: enough wavefronts to keep
// every CU's memory pipeline full, few enough that the per-workgroup atomic
// stays rare.
int tensor_grid(int64_t rows) {
    const int64_t cap = (int64_t)current_device_props().cus * 2;
    const int64_t need = (rows + kWaves - 1) / kWaves;
    return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

template <int F, bool DELAYED>
hipError_t quant_tensor_reg(int chunks, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin,
                            const float* scale, uint8_t* q, int64_t ldq, float* scale_inv, float* amax,
                            hipStream_t st) {
    const dim3 grid(tensor_grid(rows)), block(kBlock);
#define FP8_TENSOR_CASE(C)                                                                                          \
    case C:                                                                                                         \
        hipLaunchKernelGGL((k_quant_tensor_reg<F, C, DELAYED>), grid, block, 0, st, x, rows, cols, ldx, margin,     \
                           scale, q, ldq, scale_inv, amax);                                                         \
        break;
    switch (chunks) {
        FP8_TENSOR_CASE(1)
        FP8_TENSOR_CASE(2)
        FP8_TENSOR_CASE(4)
        FP8_TENSOR_CASE(8)
        FP8_TENSOR_CASE(16)
        default:
            FP8_TENSOR_CASE(32)
    }
#undef FP8_TENSOR_CASE
    return hipGetLastError();
}

template <int F>
hipError_t quant_tensor_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin,
                            const float* scale, uint8_t* q, int64_t ldq, float* scale_inv, float* amax,
                            hipStream_t st) {
    const bool vec = is_aligned(x, 16) && is_aligned(q, 8) && ldx % 8 == 0 && ldq % 8 == 0 && cols % 8 == 0;
    const int chunks = vec && rows > 0 && cols > 0 ? reg_chunks(cols) : 0;
    const dim3 grid(strided_grid(rows)), block(kBlock);
    if (chunks) {
        if (scale) return quant_tensor_reg<F, true>(chunks, x, rows, cols, ldx, margin, scale, q, ldq, scale_inv, amax, st);
        hipError_t e = launch_amax(x, rows, cols, ldx, 0, amax, st);
        if (e != hipSuccess) return e;
        return quant_tensor_reg<F, false>(chunks, x, rows, cols, ldx, margin, scale, q, ldq, scale_inv, amax, st);
    }
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
    if (n <= kDelayedFusedMax) {
        hipLaunchKernelGGL((k_delayed_update_fused<F>), dim3(1), dim3(kBlock), 0, st, cur_amax, history, head, n, L,
                           algo, margin, scale, scale_inv);
        return hipGetLastError();
    }
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
        const int chunks = vec && cols > 0 ? reg_chunks(cols) : 0;
        if (chunks) {
            const dim3 grid(grid_for_rows(rows)), block(kBlock);
#define FP8_AMAX_ROWS_CASE(C)                                                                                    \
    case C:                                                                                                      \
        hipLaunchKernelGGL((k_amax_rows_reg<C>), grid, block, 0, st, x, rows, cols, ldx, out);                   \
        break;
            switch (chunks) {
                FP8_AMAX_ROWS_CASE(1)
                FP8_AMAX_ROWS_CASE(2)
                FP8_AMAX_ROWS_CASE(4)
                FP8_AMAX_ROWS_CASE(8)
                FP8_AMAX_ROWS_CASE(16)
                default:
                    FP8_AMAX_ROWS_CASE(32)
            }
#undef FP8_AMAX_ROWS_CASE
            return hipGetLastError();
        }
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
        const int chunks = vec ? reg_chunks(cols) : 0;     // (cols > 0 here)
        if (chunks) {
            const dim3 grid(tensor_grid(rows)), block(kBlock);
#define FP8_AMAX_CASE(C)                                                                                         \
    case C:                                                                                                      \
        hipLaunchKernelGGL((k_amax_tensor_reg<C>), grid, block, 0, st, x, rows, cols, ldx, out);                 \
        break;
            switch (chunks) {
                FP8_AMAX_CASE(1)
                FP8_AMAX_CASE(2)
                FP8_AMAX_CASE(4)
                FP8_AMAX_CASE(8)
                FP8_AMAX_CASE(16)
                default:
                    FP8_AMAX_CASE(32)
            }
#undef FP8_AMAX_CASE
            return hipGetLastError();
        }
        if (vec)
            hipLaunchKernelGGL((k_amax_tensor<true>), dim3(strided_grid(rows)), dim3(kBlock), 0, st, x, rows, cols, ldx,
                               out);
        else
            hipLaunchKernelGGL((k_amax_tensor<false>), dim3(strided_grid(rows)), dim3(kBlock), 0, st, x, rows, cols,
                               ldx, out);
        return hipGetLastError();
    }
    const unsigned gy = (unsigned)((rows + kColRows - 1) / kColRows);
    if (vec) {
        // about two workgroups per CU in all, each striding over row bands
        const int64_t bands = (rows + kColAmaxRows - 1) / kColAmaxRows, chunks = (cols + 511) / 512;
        int64_t workers = (int64_t)current_device_props().cus * 2 / chunks;
        workers = workers < 1 ? 1 : (workers > bands ? bands : workers);
        hipLaunchKernelGGL(k_amax_cols_vec, dim3((unsigned)workers, (unsigned)chunks), dim3(kBlock), 0, st, x, rows,
                           cols, ldx, out);
    } else {
        hipLaunchKernelGGL(k_amax_cols_scalar, dim3(gy, (unsigned)((cols + kBlock - 1) / kBlock)), dim3(kBlock), 0, st,
                           x, rows, cols, ldx, out);
    }
    return hipGetLastError();
}

hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            uint8_t* q, int64_t ldq, float* scale_inv, float* amax_out, bool reread, hipStream_t st) {
    if (rows == 0) return hipSuccess;
#define CALL(F) quant_row_fmt<F>(x, rows, cols, ldx, margin, q, ldq, scale_inv, amax_out, reread, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

template <int F>
hipError_t quant_row_batch_fmt(const RowBatch& b, int64_t blocks, int64_t cols, int margin, hipStream_t st) {
    const int64_t per_lane = (cols / 8 + 63) / 64;
#define FP8_ROW_BATCH_CASE(C)                                                                                      \
    if (per_lane <= C) {                                                                                           \
        hipLaunchKernelGGL((k_quant_row_batch<F, C>), dim3((unsigned)blocks), dim3(kBlock), 0, st, b, cols, margin); \
        return hipGetLastError();                                                                                  \
    }
    FP8_ROW_BATCH_CASE(1)
    FP8_ROW_BATCH_CASE(2)
    FP8_ROW_BATCH_CASE(4)
    FP8_ROW_BATCH_CASE(8)
    FP8_ROW_BATCH_CASE(16)
    FP8_ROW_BATCH_CASE(32)
#undef FP8_ROW_BATCH_CASE
    return hipErrorInvalidValue;   // (the caller checked per_lane <= 32)
}

// Launch shape of the column-amax rowwise kernel by row length (16-byte
// chunks per lane): wavefronts per workgroup, workgroups per CU, running max
// in registers (REG) or folded into LDS per row, next row prefetched (PREF).
struct ColmaxShape {
    int waves, wg_per_cu;
};
ColmaxShape colmax_shape(int64_t per_lane, bool grouped) {
    if (per_lane > 8) return {4, 1};        // 16, 32 chunks: the row and its running max fill a SIMD's registers
    // grouped: one workgroup of 16 wavefronts per CU (a quarter of the
    // per-group flushes of four workgroups of 4; the MoE backward's dY,
    // 16384 x 2048: 35 -> 30 us; two rows in flight per wavefront, or two
    // workgroups of 8, were slower); rows of 8 chunks per lane would not fit
    // 16 wavefronts' registers: two workgroups of 8
    if (grouped) return per_lane > 4 ? ColmaxShape{8, 2} : ColmaxShape{16, 1};
    return {4, 4};
}
template <int F>
hipError_t quant_row_colmax_fmt(const RowBatch& b, int64_t blocks, int64_t cols, int margin, int waves,
                                bool grouped, hipStream_t st) {
    const int64_t per_lane = (cols / 8 + 63) / 64;
    // clear every requested column amax (one launch), then the single pass
    const int64_t nfill = b.cam_first[b.count];
    hipLaunchKernelGGL(k_fill_col_amax, dim3((unsigned)((nfill + kBlock - 1) / kBlock < 1024
                                                            ? (nfill + kBlock - 1) / kBlock : 1024)),
                       dim3(kBlock), 0, st, b);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
#define FP8_ROW_COLMAX_CASE(C, W, REG, PREF, GR)                                                                   \
    if (per_lane <= C && waves == W && grouped == GR) {                                                            \
        hipLaunchKernelGGL((k_quant_row_colmax<F, C, W, REG, PREF, GR>), dim3((unsigned)blocks), dim3(W * 64), 0, st, \
                           b, cols, margin);                                                                       \
        return hipGetLastError();                                                                                  \
    }
    FP8_ROW_COLMAX_CASE(1, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(2, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(4, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(8, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(16, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(32, 4, true, false, false)
    FP8_ROW_COLMAX_CASE(1, 16, true, false, true)
    FP8_ROW_COLMAX_CASE(2, 16, true, false, true)
    FP8_ROW_COLMAX_CASE(4, 16, true, false, true)
    FP8_ROW_COLMAX_CASE(8, 8, true, false, true)
    FP8_ROW_COLMAX_CASE(16, 4, true, false, true)
    FP8_ROW_COLMAX_CASE(32, 4, false, false, true)     // (a running max of 32 chunks would not fit beside the row)
#undef FP8_ROW_COLMAX_CASE
    return hipErrorInvalidValue;   // (the caller checked per_lane <= 32)
}

hipError_t launch_quant_row_batch(int count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                  const int64_t* ldx, int fmt, int margin, uint8_t* const* q, const int64_t* ldq,
                                  float* const* scale_inv, float* const* amax_out, float* const* col_amax,
                                  const int64_t* const* col_groups, const int32_t* ngroups, hipStream_t st) {
    bool any_col = false, any_grouped = false;
    for (int j = 0; j < count && col_amax; ++j) {
        any_col = any_col || col_amax[j] != nullptr;
        any_grouped = any_grouped || (col_amax[j] && ngroups && ngroups[j] > 0);
    }
    // one launch when every tensor takes the register kernel (vector layout,
    // rows of at most 32 chunks per lane); otherwise one launch per tensor
    // (and a separate column-amax pass per tensor that asks for it)
    bool one = count <= kMaxRowBatch && cols > 0 && cols % 8 == 0 && (cols / 8 + 63) / 64 <= 32;
    int64_t total_rows = 0;
    for (int j = 0; j < count && one; ++j) {
        one = is_aligned(x[j], 16) && is_aligned(q[j], 8) && ldx[j] % 8 == 0 && ldq[j] % 8 == 0;
        total_rows += rows[j];
    }
    one = one && total_rows / kWaves < ((int64_t)1 << 31) - kMaxRowBatch;    // the grid's x extent
    if (!one && any_grouped) return hipErrorInvalidValue;   // (the caller checked the layouts)
    if (!one) {
        for (int j = 0; j < count; ++j) {
            float* ca = any_col ? col_amax[j] : nullptr;
            hipError_t e = launch_quant_row(x[j], rows[j], cols, ldx[j], fmt, margin, q[j], ldq[j], scale_inv[j],
                                            amax_out ? amax_out[j] : nullptr, ca != nullptr, st);
            if (e == hipSuccess && ca) e = launch_amax(x[j], rows[j], cols, ldx[j], 2, ca, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    RowBatch b{};
    b.count = count;
    b.nt_store = streamed_codes(total_rows * cols);
    // with column amax: a few workgroups per CU in all (colmax_shape), dealt to
    // the tensors in proportion to their rows (each striding over its rows)
    const ColmaxShape shape = colmax_shape((cols / 8 + 63) / 64, any_grouped);
    const int64_t waves = shape.waves;
    const int64_t target = (int64_t)current_device_props().cus * shape.wg_per_cu;
    int64_t blocks = 0;
    for (int j = 0; j < count; ++j) {
        b.x[j] = x[j];
        b.q[j] = q[j];
        b.scale_inv[j] = scale_inv[j];
        b.amax[j] = amax_out ? amax_out[j] : nullptr;
        b.col_amax[j] = any_col ? col_amax[j] : nullptr;
        const int gj = any_col && ngroups ? ngroups[j] : 0;
        b.groups[j] = gj > 0 ? col_groups[j] : nullptr;
        b.ngroups[j] = gj > 0 ? gj : 0;
        b.cam_first[j + 1] = b.cam_first[j] + cols * (gj > 0 ? gj : 1);
        b.rows[j] = rows[j];
        b.ldx[j] = ldx[j];
        b.ldq[j] = ldq[j];
        b.first[j] = blocks;
        const int64_t need = (rows[j] + (any_col ? waves : kWaves) - 1) / (any_col ? waves : kWaves);
        if (any_col) {
            int64_t share = total_rows > 0 ? (target * rows[j] + total_rows - 1) / total_rows : 0;
            share = share < 1 ? 1 : share;
            blocks += need < share ? need : share;
        } else {
            blocks += need;
        }
    }
    for (int j = count; j <= kMaxRowBatch; ++j) b.first[j] = blocks;
    for (int j = count + 1; j <= kMaxRowBatch; ++j) b.cam_first[j] = b.cam_first[count];
    if (any_col) {
        switch (fmt) {
            case kE4M3: return quant_row_colmax_fmt<kE4M3>(b, blocks, cols, margin, (int)waves, any_grouped, st);
            case kE5M2: return quant_row_colmax_fmt<kE5M2>(b, blocks, cols, margin, (int)waves, any_grouped, st);
            case kE4M3Fnuz: return quant_row_colmax_fmt<kE4M3Fnuz>(b, blocks, cols, margin, (int)waves, any_grouped, st);
            default: return quant_row_colmax_fmt<kE5M2Fnuz>(b, blocks, cols, margin, (int)waves, any_grouped, st);
        }
    }
    if (blocks == 0) return hipSuccess;
    switch (fmt) {
        case kE4M3: return quant_row_batch_fmt<kE4M3>(b, blocks, cols, margin, st);
        case kE5M2: return quant_row_batch_fmt<kE5M2>(b, blocks, cols, margin, st);
        case kE4M3Fnuz: return quant_row_batch_fmt<kE4M3Fnuz>(b, blocks, cols, margin, st);
        default: return quant_row_batch_fmt<kE5M2Fnuz>(b, blocks, cols, margin, st);
    }
}

hipError_t launch_quant_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            int transpose, uint8_t* qt, int64_t ldqt, float* scale_inv, const float* col_amax,
                            hipStream_t st) {
    if (cols == 0) return hipSuccess;
    if (rows == 0) {
        // no rows: every column has amax 0 (already in col_amax) -> scale 1
        return launch_fill(scale_inv, cols, 1.0f, st);
    }
#define CALL(F) quant_col_fmt<F>(x, rows, cols, ldx, margin, transpose, qt, ldqt, scale_inv, col_amax, st)
    switch (fmt) {
        case kE4M3: return CALL(kE4M3);
        case kE5M2: return CALL(kE5M2);
        case kE4M3Fnuz: return CALL(kE4M3Fnuz);
        default: return CALL(kE5M2Fnuz);
    }
#undef CALL
}

template <int F>
hipError_t quant_rowcol_fmt(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int margin, uint8_t* q,
                            int64_t ldq, float* row_scale_inv, float* row_amax, uint8_t* qt, int64_t ldqt,
                            float* col_scale_inv, float* col_amax, hipStream_t st) {
    const int vec_store = is_aligned(qt, 16) && ldqt % 16 == 0;
    const dim3 grid((unsigned)((rows + kColTileR - 1) / kColTileR), (unsigned)((cols + kColTileC - 1) / kColTileC));
    hipLaunchKernelGGL((k_quant_rowcol_tiled<F>), grid, dim3(kBlock), 0, st, x, rows, cols, ldx, margin, q, ldq,
                       row_scale_inv, row_amax, qt, ldqt, col_scale_inv, col_amax, vec_store);
    return hipGetLastError();
}

hipError_t launch_quant_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                               uint8_t* q, int64_t ldq, float* row_scale_inv, float* row_amax, uint8_t* qt,
                               int64_t ldqt, float* col_scale_inv, float* col_amax, hipStream_t st) {
    if (rows == 0 || cols == 0) {
        hipError_t e = launch_fill(col_amax, cols, 0.0f, st);
        if (e == hipSuccess) e = launch_fill(col_scale_inv, cols, 1.0f, st);
        return e;
    }
    // first pass: both amax (cleared first), then the dual cast
    hipError_t e = launch_fill(row_amax, rows, 0.0f, st);
    if (e == hipSuccess) e = launch_fill(col_amax, cols, 0.0f, st);
    if (e != hipSuccess) return e;
    const int64_t bands = (rows + kColAmaxRows - 1) / kColAmaxRows, chunks = (cols + 511) / 512;
    int64_t workers = (int64_t)current_device_props().cus * 2 / chunks;
    workers = workers < 1 ? 1 : (workers > bands ? bands : workers);
    hipLaunchKernelGGL(k_amax_rows_cols_vec, dim3((unsigned)workers, (unsigned)chunks), dim3(kBlock), 0, st, x, rows,
                       cols, ldx, row_amax, col_amax);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
#define CALL(F) quant_rowcol_fmt<F>(x, rows, cols, ldx, margin, q, ldq, row_scale_inv, row_amax, qt, ldqt, col_scale_inv, \
                                    col_amax, st)
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

template <int F>
hipError_t quant_tensor_batch_fmt(const TensorBatch& b, int64_t blocks, int64_t cols, hipStream_t st) {
    switch (reg_chunks(cols)) {
#define FP8_TENSOR_BATCH_CASE(C)                                                                                   \
    case C:                                                                                                        \
        hipLaunchKernelGGL((k_quant_tensor_batch<F, C>), dim3((unsigned)blocks), dim3(kBlock), 0, st, b, cols);    \
        break;
        FP8_TENSOR_BATCH_CASE(1)
        FP8_TENSOR_BATCH_CASE(2)
        FP8_TENSOR_BATCH_CASE(4)
        FP8_TENSOR_BATCH_CASE(8)
        FP8_TENSOR_BATCH_CASE(16)
        default:
            FP8_TENSOR_BATCH_CASE(32)
#undef FP8_TENSOR_BATCH_CASE
    }
    return hipGetLastError();
}

hipError_t launch_quant_tensor_batch(int count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                     const int64_t* ldx, int fmt, const float* const* scale, uint8_t* const* q,
                                     const int64_t* ldq, float* const* scale_inv, float* const* amax,
                                     hipStream_t st) {
    // one launch when every tensor takes the register kernel; otherwise one per tensor
    bool one = count <= kMaxRowBatch && cols > 0 && cols % 8 == 0 && reg_chunks(cols) > 0;
    for (int j = 0; j < count && one; ++j)
        one = rows[j] > 0 && is_aligned(x[j], 16) && is_aligned(q[j], 8) && ldx[j] % 8 == 0 && ldq[j] % 8 == 0;
    if (!one) {
        for (int j = 0; j < count; ++j) {
            const hipError_t e = launch_quant_tensor(x[j], rows[j], cols, ldx[j], fmt, 0, scale[j], q[j], ldq[j],
                                                     scale_inv[j], amax[j], st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    TensorBatch b{};
    b.count = count;
    int64_t blocks = 0;
    for (int j = 0; j < count; ++j) {
        b.x[j] = x[j];
        b.q[j] = q[j];
        b.scale[j] = scale[j];
        b.scale_inv[j] = scale_inv[j];
        b.amax[j] = amax[j];
        b.rows[j] = rows[j];
        b.ldx[j] = ldx[j];
        b.ldq[j] = ldq[j];
        b.first[j] = blocks;
        blocks += tensor_grid(rows[j]);
    }
    for (int j = count; j <= kMaxRowBatch; ++j) b.first[j] = blocks;
    switch (fmt) {
        case kE4M3: return quant_tensor_batch_fmt<kE4M3>(b, blocks, cols, st);
        case kE5M2: return quant_tensor_batch_fmt<kE5M2>(b, blocks, cols, st);
        case kE4M3Fnuz: return quant_tensor_batch_fmt<kE4M3Fnuz>(b, blocks, cols, st);
        default: return quant_tensor_batch_fmt<kE5M2Fnuz>(b, blocks, cols, st);
    }
}

hipError_t launch_mx_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                               int64_t ldq, uint8_t* scale, int64_t ld_scale, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int chunks = reg_chunks(cols < kMxSlice ? cols : kMxSlice);
    const unsigned slices = (unsigned)((cols + kMxSlice - 1) / kMxSlice);
    // rows of up to 8 chunks per lane: 16 rows (wavefronts) per workgroup, two
    // workgroups per CU; longer rows: 4 (16 wavefronts of 16-chunk rows would
    // leave one workgroup per CU: slower)
#define FP8_MX_CASE(F, C)                                                                                        \
    case C: {                                                                                                    \
        constexpr int W = C <= 8 ? 16 : 4;                                                                       \
        hipLaunchKernelGGL((k_mx_quant_row<F, C, W>), dim3((unsigned)((rows + W - 1) / W), slices), dim3(W * 64), \
                           0, st, x, rows, cols, ldx, q, ldq, scale, ld_scale);                                  \
        break;                                                                                                   \
    }
#define FP8_MX_FMT(F)                                                                                            \
    switch (chunks) {                                                                                            \
        FP8_MX_CASE(F, 1)                                                                                        \
        FP8_MX_CASE(F, 2)                                                                                        \
        FP8_MX_CASE(F, 4)                                                                                        \
        FP8_MX_CASE(F, 8)                                                                                        \
        FP8_MX_CASE(F, 16)                                                                                       \
        default:                                                                                                 \
            FP8_MX_CASE(F, 32)                                                                                   \
    }
    if (fmt == kE4M3) {
        FP8_MX_FMT(kE4M3)
    } else {
        FP8_MX_FMT(kE5M2)
    }
#undef FP8_MX_FMT
#undef FP8_MX_CASE
    return hipGetLastError();
}

hipError_t launch_blockwise_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int weight,
                                  uint8_t* q, int64_t ldq, uint8_t* scale, int64_t ld_scale, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (weight) {
        const int64_t rt = (rows + 127) / 128, kbs = cols / 128;
        const int kfast = rt <= 65535;
        const dim3 grid(kfast ? (unsigned)kbs : (unsigned)rt, kfast ? (unsigned)rt : (unsigned)kbs), block(kBlock);
        if (fmt == kE4M3)
            hipLaunchKernelGGL((k_blockwise_quant_weight<kE4M3>), grid, block, 0, st, x, rows, ldx, q, ldq, scale,
                               ld_scale, kfast);
        else
            hipLaunchKernelGGL((k_blockwise_quant_weight<kE5M2>), grid, block, 0, st, x, rows, ldx, q, ldq, scale,
                               ld_scale, kfast);
        return hipGetLastError();
    }
    const int chunks = reg_chunks(cols < kMxSlice ? cols : kMxSlice);
    const unsigned slices = (unsigned)((cols + kMxSlice - 1) / kMxSlice);
#define FP8_BW_CASE(F, C)                                                                                        \
    case C: {                                                                                                    \
        constexpr int W = C <= 8 ? 16 : 4;                                                                       \
        hipLaunchKernelGGL((k_blockwise_quant_act<F, C, W>), dim3((unsigned)((rows + W - 1) / W), slices),       \
                           dim3(W * 64), 0, st, x, rows, cols, ldx, q, ldq, scale, ld_scale);                    \
        break;                                                                                                   \
    }
#define FP8_BW_FMT(F)                                                                                            \
    switch (chunks) {                                                                                            \
        FP8_BW_CASE(F, 1)                                                                                        \
        FP8_BW_CASE(F, 2)                                                                                        \
        FP8_BW_CASE(F, 4)                                                                                        \
        FP8_BW_CASE(F, 8)                                                                                        \
        FP8_BW_CASE(F, 16)                                                                                       \
        default:                                                                                                 \
            FP8_BW_CASE(F, 32)                                                                                   \
    }
    if (fmt == kE4M3) {
        FP8_BW_FMT(kE4M3)
    } else {
        FP8_BW_FMT(kE5M2)
    }
#undef FP8_BW_FMT
#undef FP8_BW_CASE
    return hipGetLastError();
}

hipError_t launch_grouped_quant_col(const uint16_t* x, int64_t total_m, int64_t cols, int64_t ldx, int fmt,
                                    int margin, const int64_t* offsets, int g, uint8_t* qt, int64_t ldqt,
                                    float* scale_inv, float* col_amax, int col_amax_ready, hipStream_t st) {
    if (cols == 0) return hipSuccess;
    hipError_t e = hipSuccess;
    // Groups of at most kSmallGroupRows rows in one pass, when the tensor is
    // larger than the 256 MB last-level cache (the two-pass path's second read
    // then comes from HBM: the MoE backward's expert weights, 940 MB, 483 -> 402 us); a
    // tensor that fits is read the second time from that cache, and the
    // two-pass path is faster (its token-side tensors, 67 and 235 MB: 52 / 167 us
    // against 115 / 307 us one-pass). Not with a supplied amax.
    const int small = !col_amax_ready && (cols + kSmallStrip - 1) / kSmallStrip <= 65535 &&
                      total_m * cols * 2 > ((int64_t)256 << 20);
    if (!col_amax_ready) {
        e = launch_fill(col_amax, (int64_t)g * cols, 0.0f, st);
        if (e != hipSuccess) return e;
        if (small) {
            const dim3 sgrid((unsigned)g, (unsigned)((cols + kSmallStrip - 1) / kSmallStrip));
            switch (fmt) {
                case kE4M3:
                    hipLaunchKernelGGL((k_grouped_quant_col_small<kE4M3>), sgrid, dim3(kBlock), 0, st, x, total_m,
                                       cols, ldx, margin, offsets, g, qt, ldqt, scale_inv, col_amax);
                    break;
                case kE5M2:
                    hipLaunchKernelGGL((k_grouped_quant_col_small<kE5M2>), sgrid, dim3(kBlock), 0, st, x, total_m,
                                       cols, ldx, margin, offsets, g, qt, ldqt, scale_inv, col_amax);
                    break;
                case kE4M3Fnuz:
                    hipLaunchKernelGGL((k_grouped_quant_col_small<kE4M3Fnuz>), sgrid, dim3(kBlock), 0, st, x,
                                       total_m, cols, ldx, margin, offsets, g, qt, ldqt, scale_inv, col_amax);
                    break;
                default:
                    hipLaunchKernelGGL((k_grouped_quant_col_small<kE5M2Fnuz>), sgrid, dim3(kBlock), 0, st, x,
                                       total_m, cols, ldx, margin, offsets, g, qt, ldqt, scale_inv, col_amax);
                    break;
            }
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (total_m > 0) {
            hipLaunchKernelGGL(k_grouped_amax_cols,
                               dim3((unsigned)((total_m + kColAmaxRows - 1) / kColAmaxRows), (unsigned)((cols + 511) / 512)),
                               dim3(kBlock), 0, st, x, total_m, cols, ldx, offsets, g, col_amax, small);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    const int64_t n = (int64_t)g * cols;
    const unsigned sblocks = (unsigned)((n + kBlock - 1) / kBlock < 1024 ? (n + kBlock - 1) / kBlock : 1024);
    // every group's padded tile count is at most m_g / 128 + 2
    // row-tile slots: the tile count's upper bound, at most about eight
    // workgroups per CU over the column tiles (each workgroup forms the group
    // prefix sums once and strides over row tiles)
    const int64_t ctiles = (cols + kColTileC - 1) / kColTileC;
    const int64_t rt_bound = (total_m + kColTileR - 1) / kColTileR + 2 * (int64_t)g;
    const int64_t rt_cap = ((int64_t)current_device_props().cus * 8 + ctiles - 1) / ctiles;
    const dim3 grid((unsigned)(rt_bound < rt_cap ? rt_bound : rt_cap), (unsigned)ctiles);
    // the cast also writes scale_inv (each group's first row tile; the empty
    // groups by the first row-tile slot); with no rows only scale_inv is left
#define CALL(F)                                                                                                  \
    do {                                                                                                         \
        if (total_m > 0)                                                                                         \
            hipLaunchKernelGGL((k_grouped_quant_col_tiled<F>), grid, dim3(kBlock), 0, st, x, total_m, cols, ldx, \
                               margin, offsets, g, qt, ldqt, col_amax, scale_inv, 1, small);                     \
        else                                                                                                     \
            hipLaunchKernelGGL((k_scale_inv_from_amax<F>), dim3(sblocks), dim3(kBlock), 0, st, col_amax, n,      \
                               margin, scale_inv);                                                               \
    } while (0)
    switch (fmt) {
        case kE4M3: CALL(kE4M3); break;
        case kE5M2: CALL(kE5M2); break;
        case kE4M3Fnuz: CALL(kE4M3Fnuz); break;
        default: CALL(kE5M2Fnuz); break;
    }
#undef CALL
    return hipGetLastError();
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
