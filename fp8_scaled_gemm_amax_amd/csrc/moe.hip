// moe.hip - the memory-bound steps of the MoE layer's forward around its two
// grouped GEMMs: routing (expert-sorted order), the token permutation fused
// with the rowwise cast, SwiGLU fused with the rowwise cast, and the weighted
// combine back to token order.
//
// Sources: "How PyTorch FP8 Optimizations on AMD GPUs Reduce LLM Cost and Scale
// Training Past 1,000 GPUs", What Happened (the per-MoE-layer latency);
// "FP8 Training on AMD GPUs with TorchTitan and TorchAO" (fused quantization
// kernels, FP8 grouped GEMM for MoE). The pages do not define the layer; the
// reading here is the plain top-k MoE feed-forward layer with SwiGLU experts.
//
// Layout choices for CDNA4: one 64-lane wavefront per token row (row in
// registers, 16-byte loads, 8-byte code stores); the permutation writes each
// token's codes straight to its k expert rows, so no bf16 permuted copy ever
// reaches HBM; the SwiGLU output is cast from fp32 registers, never stored.
#include "fp8_device.hpp"
#include "kernels.hpp"

namespace fp8amax {
namespace {

constexpr int kBlock = 256;   // 4 wavefronts
constexpr int kWaves = kBlock / 64;

// ---------------------------------------------------------------- routing --
// One workgroup of 16 wavefronts walks the T*k entries in chunks of 1024, in
// (token, slot) order. Within a wavefront, entries of one expert get their
// rank by ballots (one round per distinct expert present) and the leader
// writes the wavefront's count of that expert to LDS; then one thread per
// expert turns the 16 wavefronts' counts into running offsets (earlier chunks
// + earlier wavefronts), so an entry's row within its expert is one LDS read
// + its rank: the stable counting sort, deterministic. The counts are double
// buffered (the expert threads clear the other buffer), so a chunk costs two
// barriers. The expert offsets are the exclusive scan of the totals. Entries
// are read in batches of 16 chunks held in registers (all loads of a batch in
// flight at once); when everything fits one batch, the rows are completed in
// registers and written once, else each batch writes its rows within the
// expert and a last pass adds the offsets. Entries whose expert index is
// outside [0, E) get dest = -1, not counted.
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteBatch = 16;                             // chunks per batch
constexpr int64_t kRouteBatchEntries = (int64_t)kRouteThreads * kRouteBatch;

__global__ __launch_bounds__(kRouteThreads) void k_moe_route(const int32_t* __restrict__ idx, int64_t n, int E,
                                                               int64_t* __restrict__ offsets,
                                                               int32_t* __restrict__ dest) {
    __shared__ int32_t run[kMoeMaxExperts];                      // entries of each expert in earlier chunks
    __shared__ int32_t wcnt[2][kRouteWaves][kMoeMaxExperts];     // per wavefront: count, then running offset
    __shared__ int32_t wsum[kRouteWaves];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int e = tid; e < E; e += kRouteThreads) {
        run[e] = 0;
#pragma unroll
        for (int v = 0; v < kRouteWaves; ++v) wcnt[0][v][e] = wcnt[1][v][e] = 0;
    }
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    const bool one_batch = n <= kRouteBatchEntries;
    int ev[kRouteBatch], pos[kRouteBatch];
    int buf = 0;
    for (int64_t b0 = 0; b0 < n; b0 += kRouteBatchEntries) {
#pragma unroll
        for (int c = 0; c < kRouteBatch; ++c) {
            const int64_t i = b0 + (int64_t)c * kRouteThreads + tid;
            const int e = i < n ? idx[i] : -1;
            ev[c] = (e >= 0 && e < E) ? e : -1;
        }
#pragma unroll
        for (int c = 0; c < kRouteBatch; ++c) {
            int32_t(*cnt)[kMoeMaxExperts] = wcnt[buf];
            const int e = ev[c];
            uint64_t pending = __ballot(e >= 0);
            int rank = 0;
            while (pending) {                                    // uniform over the wavefront
                const int leader = __ffsll((unsigned long long)pending) - 1;
                const int e0 = __builtin_amdgcn_readlane(e, leader);
                const uint64_t m = __ballot(e == e0);
                if (e == e0) rank = __popcll(m & below);
                if (lane == leader) cnt[w][e0] = __popcll(m);
                pending &= ~m;
            }
            __syncthreads();
            for (int ee = tid; ee < E; ee += kRouteThreads) {   // counts -> running offsets
                int c16[kRouteWaves];
#pragma unroll
                for (int v = 0; v < kRouteWaves; ++v) c16[v] = cnt[v][ee];
                int acc = run[ee];
#pragma unroll
                for (int v = 0; v < kRouteWaves; ++v) {
                    cnt[v][ee] = acc;
                    acc += c16[v];
                    wcnt[buf ^ 1][v][ee] = 0;
                }
                run[ee] = acc;
            }
            __syncthreads();
            pos[c] = e >= 0 ? cnt[w][e] + rank : -1;             // row within the expert
            buf ^= 1;
        }
        if (!one_batch) {
#pragma unroll
            for (int c = 0; c < kRouteBatch; ++c) {
                const int64_t i = b0 + (int64_t)c * kRouteThreads + tid;
                if (i < n) dest[i] = pos[c];
            }
        }
    }
    __syncthreads();                                             // (every pos read done before pre reuses LDS)
    // exclusive scan of run[0 .. E) (E <= 1024: one expert per thread)
    const int mine = tid < E ? run[tid] : 0;
    int incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int excl = incl - mine;
    for (int v = 0; v < w; ++v) excl += wsum[v];
    int32_t* pre = &wcnt[0][0][0];                          // (the counts are dead)
    if (tid < E) {
        pre[tid] = excl;
        offsets[tid] = excl;
    }
    if (tid == E - 1) offsets[E] = excl + mine;
    __syncthreads();
    if (one_batch) {
#pragma unroll
        for (int c = 0; c < kRouteBatch; ++c) {
            const int64_t i = (int64_t)c * kRouteThreads + tid;
            if (i < n) dest[i] = ev[c] >= 0 ? pre[ev[c]] + pos[c] : -1;
        }
    } else {
        for (int64_t i = tid; i < n; i += kRouteThreads) {
            const int e = idx[i];
            if (e >= 0 && e < E) dest[i] += pre[e];
        }
    }
}

// ------------------------------------------------- permutation + rowwise cast --
// One wavefront per token: the row in registers, its amax and scale, the codes
// encoded once and stored to each of the token's k destination rows (with the
// row's scale_inv). Destinations outside [0, rows_out) are skipped.
template <int F, int MAXC>
__global__ __launch_bounds__(kBlock) void k_moe_permute_quant_row(const uint16_t* __restrict__ x, int64_t tokens,
                                                                  int64_t cols, int64_t ldx,
                                                                  const int32_t* __restrict__ dest, int topk,
                                                                  int64_t rows_out, int margin,
                                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                                  float* __restrict__ scale_inv) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= tokens) return;
    const int nch = (int)(cols >> 3);
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * ldx);
    uint4 v[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        v[c] = load_stream(xr + (ch < nch ? ch : nch - 1));  // past the row: a duplicate chunk, never stored
    }
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) mx = word_absmax(mx, v[c]);
    const float amax = amax_from_bits16(wave_max_u32(pk_fold(mx)));
    const float s = scale_from_amax<F>(amax, margin);
    uint2 code[MAXC];
    if (!__builtin_isnan(amax)) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) code[c] = encode8<F, true>(v[c], s);
    } else {   // a NaN in the row (then s = 1): the bit-level encoder keeps NaN signs
#pragma unroll
        for (int c = 0; c < MAXC; ++c) code[c] = encode8<F, false>(v[c], s);
    }
    const float si = 1.0f / s;
    for (int j = 0; j < topk; ++j) {
        const int64_t d = dest[t * topk + j];
        if (d < 0 || d >= rows_out) continue;               // uniform over the wavefront
        uint2* qr = reinterpret_cast<uint2*>(q + d * ldq);
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = lane + c * 64;
            if (ch < nch) qr[ch] = code[c];
        }
        if (lane == 0) scale_inv[d] = si;
    }
}

// ------------------------------------------------------- SwiGLU + rowwise cast --
// Row r of h holds gate (columns 0 .. I-1) and up (I .. 2I-1), bf16. One
// wavefront per row: a = silu(gate) * up in fp32 registers, the row's amax over
// the fp32 magnitudes (bit patterns: NaN above Inf), the scale, the cast.
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

template <int F, int MAXC>
__global__ __launch_bounds__(kBlock) void k_swiglu_quant_row(const uint16_t* __restrict__ h, int64_t rows,
                                                             int64_t inter, int64_t ldh, int margin,
                                                             uint8_t* __restrict__ q, int64_t ldq,
                                                             float* __restrict__ scale_inv) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int nch = (int)(inter >> 3);
    const uint4* gr = reinterpret_cast<const uint4*>(h + row * ldh);
    const uint4* ur = reinterpret_cast<const uint4*>(h + row * ldh + inter);
    uint4 gv[MAXC], uv[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        const int cc = ch < nch ? ch : nch - 1;             // past the row: a duplicate chunk, never stored
        gv[c] = load_stream(gr + cc);
        uv[c] = load_stream(ur + cc);
    }
    float a[MAXC][8];
    uint32_t mxb = 0;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const uint32_t gw[4] = {gv[c].x, gv[c].y, gv[c].z, gv[c].w};
        const uint32_t uw[4] = {uv[c].x, uv[c].y, uv[c].z, uv[c].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            a[c][2 * p] = silu_f32(bf16_lo(gw[p])) * bf16_lo(uw[p]);
            a[c][2 * p + 1] = silu_f32(bf16_hi(gw[p])) * bf16_hi(uw[p]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = __float_as_uint(a[c][e]) & 0x7fffffffu;
            mxb = b > mxb ? b : mxb;
        }
    }
    const float amax = __uint_as_float(wave_max_u32(mxb));
    const float s = scale_from_amax<F>(amax, margin);
    if (lane == 0) scale_inv[row] = 1.0f / s;
    uint2* qr = reinterpret_cast<uint2*>(q + row * ldq);
    const bool nan_free = !__builtin_isnan(amax);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
        const int ch = lane + c * 64;
        uint2 o;
        if (nan_free) {
            o.x = encode4<F, true>(a[c][0] * s, a[c][1] * s, a[c][2] * s, a[c][3] * s);
            o.y = encode4<F, true>(a[c][4] * s, a[c][5] * s, a[c][6] * s, a[c][7] * s);
        } else {
            o.x = encode4<F, false>(a[c][0] * s, a[c][1] * s, a[c][2] * s, a[c][3] * s);
            o.y = encode4<F, false>(a[c][4] * s, a[c][5] * s, a[c][6] * s, a[c][7] * s);
        }
        if (ch < nch) qr[ch] = o;
    }
}

// ------------------------------------------------------- unpermute + combine --
// out[t] = bf16( sum over slots j = 0 .. k-1, in order, of w[t, j] * y[dest[t, j]] )
// accumulated in fp32. One wavefront per (token, slice of kCombineCols
// columns): 4 chunks of 8 columns per lane. Slots whose destination is outside
// [0, rows) add nothing.
constexpr int kCombineCols = 64 * 8 * 4;

__global__ __launch_bounds__(kBlock) void k_moe_unpermute_combine(const uint16_t* __restrict__ y, int64_t rows,
                                                                  int64_t cols, int64_t ldy,
                                                                  const int32_t* __restrict__ dest,
                                                                  const float* __restrict__ wts, int64_t tokens,
                                                                  int topk, uint16_t* __restrict__ out, int64_t ldo) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (t >= tokens) return;
    const int64_t c0 = (int64_t)blockIdx.y * kCombineCols;
    const int nch = (int)((cols - c0 < kCombineCols ? cols - c0 : kCombineCols) >> 3);
    float acc[4][8];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = 0.0f;
    for (int j = 0; j < topk; ++j) {
        const int64_t d = dest[t * topk + j];
        const float wj = wts[t * topk + j];
        if (d < 0 || d >= rows) continue;                   // uniform over the wavefront
        const uint4* yr = reinterpret_cast<const uint4*>(y + d * ldy + c0);
        uint4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int ch = lane + c * 64;
            v[c] = load_stream(yr + (ch < nch ? ch : nch - 1));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t yw[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                acc[c][2 * p] += wj * bf16_lo(yw[p]);
                acc[c][2 * p + 1] += wj * bf16_hi(yw[p]);
            }
        }
    }
    uint4* orow = reinterpret_cast<uint4*>(out + t * ldo + c0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int ch = lane + c * 64;
        uint4 o;
        o.x = f32_to_bf16(acc[c][0]) | (f32_to_bf16(acc[c][1]) << 16);
        o.y = f32_to_bf16(acc[c][2]) | (f32_to_bf16(acc[c][3]) << 16);
        o.z = f32_to_bf16(acc[c][4]) | (f32_to_bf16(acc[c][5]) << 16);
        o.w = f32_to_bf16(acc[c][6]) | (f32_to_bf16(acc[c][7]) << 16);
        if (ch < nch) orow[ch] = o;
    }
}

// 16-byte chunks per lane that hold a row of `cols` bf16 values (1, 2, 4, ..,
// max_c), or 0 if the row is longer.
int chunks_for(int64_t cols, int max_c) {
    const int64_t per_lane = (cols / 8 + 63) / 64;
    for (int c = 1; c <= max_c; c *= 2)
        if (per_lane <= c) return c;
    return 0;
}

unsigned grid_rows(int64_t rows) { return (unsigned)((rows + kWaves - 1) / kWaves); }

}  // namespace

hipError_t launch_moe_route(const int32_t* idx, int64_t tokens, int topk, int num_experts, int64_t* offsets,
                            int32_t* dest, hipStream_t st) {
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(kRouteThreads), 0, st, idx, tokens * topk, num_experts, offsets,
                       dest);
    return hipGetLastError();
}

hipError_t launch_moe_permute_quant_row(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ldx,
                                        const int32_t* dest, int topk, int64_t rows_out, int fmt, int margin,
                                        uint8_t* q, int64_t ldq, float* scale_inv, hipStream_t st) {
    if (tokens == 0 || cols == 0) return hipSuccess;
    const int chunks = chunks_for(cols, 32);
    if (chunks == 0) return hipErrorInvalidValue;           // (the API bounds cols)
    const dim3 grid(grid_rows(tokens)), block(kBlock);
#define FP8_PQ_CASE(F, C)                                                                                      \
    case C:                                                                                                    \
        hipLaunchKernelGGL((k_moe_permute_quant_row<F, C>), grid, block, 0, st, x, tokens, cols, ldx, dest,    \
                           topk, rows_out, margin, q, ldq, scale_inv);                                         \
        break;
#define FP8_PQ_FMT(F)                                                                                          \
    switch (chunks) {                                                                                          \
        FP8_PQ_CASE(F, 1)                                                                                      \
        FP8_PQ_CASE(F, 2)                                                                                      \
        FP8_PQ_CASE(F, 4)                                                                                      \
        FP8_PQ_CASE(F, 8)                                                                                      \
        FP8_PQ_CASE(F, 16)                                                                                     \
        default:                                                                                               \
            FP8_PQ_CASE(F, 32)                                                                                 \
    }
    switch (fmt) {
        case kE4M3: FP8_PQ_FMT(kE4M3) break;
        case kE5M2: FP8_PQ_FMT(kE5M2) break;
        case kE4M3Fnuz: FP8_PQ_FMT(kE4M3Fnuz) break;
        default: FP8_PQ_FMT(kE5M2Fnuz) break;
    }
#undef FP8_PQ_FMT
#undef FP8_PQ_CASE
    return hipGetLastError();
}

hipError_t launch_swiglu_quant_row(const uint16_t* h, int64_t rows, int64_t inter, int64_t ldh, int fmt, int margin,
                                   uint8_t* q, int64_t ldq, float* scale_inv, hipStream_t st) {
    if (rows == 0 || inter == 0) return hipSuccess;
    const int chunks = chunks_for(inter, kSwigluMaxChunks);
    if (chunks == 0) return hipErrorInvalidValue;           // (the API bounds inter)
    const dim3 grid(grid_rows(rows)), block(kBlock);
#define FP8_SW_CASE(F, C)                                                                                      \
    case C:                                                                                                    \
        hipLaunchKernelGGL((k_swiglu_quant_row<F, C>), grid, block, 0, st, h, rows, inter, ldh, margin, q, ldq, \
                           scale_inv);                                                                         \
        break;
#define FP8_SW_FMT(F)                                                                                          \
    switch (chunks) {                                                                                          \
        FP8_SW_CASE(F, 1)                                                                                      \
        FP8_SW_CASE(F, 2)                                                                                      \
        FP8_SW_CASE(F, 4)                                                                                      \
        default:                                                                                               \
            FP8_SW_CASE(F, 8)                                                                                  \
    }
    switch (fmt) {
        case kE4M3: FP8_SW_FMT(kE4M3) break;
        case kE5M2: FP8_SW_FMT(kE5M2) break;
        case kE4M3Fnuz: FP8_SW_FMT(kE4M3Fnuz) break;
        default: FP8_SW_FMT(kE5M2Fnuz) break;
    }
#undef FP8_SW_FMT
#undef FP8_SW_CASE
    return hipGetLastError();
}

hipError_t launch_moe_unpermute_combine(const uint16_t* y, int64_t rows, int64_t cols, int64_t ldy,
                                        const int32_t* dest, const float* wts, int64_t tokens, int topk,
                                        uint16_t* out, int64_t ldo, hipStream_t st) {
    if (tokens == 0 || cols == 0) return hipSuccess;
    const dim3 grid(grid_rows(tokens), (unsigned)((cols + kCombineCols - 1) / kCombineCols)), block(kBlock);
    hipLaunchKernelGGL(k_moe_unpermute_combine, grid, block, 0, st, y, rows, cols, ldy, dest, wts, tokens, topk, out,
                       ldo);
    return hipGetLastError();
}

}  // namespace fp8amax
