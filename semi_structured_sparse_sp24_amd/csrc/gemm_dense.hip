// gemm_dense.hip -- dense GEMM baseline Y = X * W^T on gfx950 MFMA.
//
// The baseline every sparse tactic is timed against and the target of every
// fallback ("Production 2:4 Structured Sparsity for LLMs", sections "Sparse
// Tactic Audit" and "Dense Fallback and Hybrid Sparsity Design").  It has
// the same two constructions, and the same split between them, as the sparse
// kernels so that the comparison is between kernels of the same design:
//   skinny  few rows of X (<= 16, or <= 64 on a narrow output): the
//           workgroup owns 16 rows of W and all of X; waves split K;
//           v_mfma_f32_16x16x32 (16-bit, two per 64-K step) or
//           v_mfma_scale_f32_16x16x128_f8f6f4 (fp8, unit scales); 5 to 16
//           rows of X staged in LDS as the sparse decode kernel does;
//   tiles   everything else: the LDS-staged tile kernels of
//           gemm_dense_big.hip.
// D is computed with A = W (rows N) and B = X (rows M), i.e. the tile of
// Y^T, and stored transposed.
#include "mfma_ops.h"

namespace sp24 {
namespace {

// 16x16 output, one "step" of dense K: 64 (16-bit) or 128 (fp8).  A lane
// (row l%16, group kg = l/16) supplies 16 bytes at byte offsets o0(kg) and
// o1(kg) of the row's step; B likewise.  The instructions only need A and B
// to assign K identically to (lane group, slot), which they do here.
template <sp24_dtype DT>
struct DenseOp16;

template <>
struct DenseOp16<SP24_BF16> {
    static constexpr int KSTEP = 64, ELEM = 2;
    __device__ static __forceinline__ f32x4 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0),
                                                    __builtin_bit_cast(bf16x8, b0), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1),
                                                       __builtin_bit_cast(bf16x8, b1), c, 0, 0, 0);
    }
};
template <>
struct DenseOp16<SP24_F16> {
    static constexpr int KSTEP = 64, ELEM = 2;
    __device__ static __forceinline__ f32x4 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a0),
                                                   __builtin_bit_cast(f16x8, b0), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1),
                                                      __builtin_bit_cast(f16x8, b1), c, 0, 0, 0);
    }
};
// int8: two v_mfma_i32_16x16x64_i8 per 128-K step (lane l: row l%16, 16
// bytes of K at 16*(l/16) of each half); int32 accumulation in the
// accumulator registers' bits, converted after the K loop.
template <>
struct DenseOp16<SP24_I8> {
    static constexpr int KSTEP = 128, ELEM = 1;
    __device__ static __forceinline__ f32x4 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
        i32x4 ci = __builtin_bit_cast(i32x4, c);
        ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a0), __builtin_bit_cast(i32x4, b0),
                                                   ci, 0, 0, 0);
        ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a1), __builtin_bit_cast(i32x4, b1),
                                                   ci, 0, 0, 0);
        return __builtin_bit_cast(f32x4, ci);
    }
};
template <>
struct DenseOp16<SP24_E4M3> {
    static constexpr int KSTEP = 128, ELEM = 1;
    __device__ static __forceinline__ f32x4 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
        struct { uint4 x, y; } aa = {a0, a1}, bb = {b0, b1};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            __builtin_bit_cast(i32x8, aa), __builtin_bit_cast(i32x8, bb), c, 0, 0, 0, 0x7f, 0, 0x7f);
    }
};

// ------------------------------------------------------------------ skinny
constexpr int kMaxWaves = 16;

// MT: 16-row blocks of X per pass; U: K steps per load batch; AT: 16-row
// tiles of W per workgroup (2 halves the X traffic per W byte, as in the
// sparse decode kernel).
template <sp24_dtype DT, sp24_dtype OUT, int MT, int U, int AT>
__global__ void __launch_bounds__(kMaxWaves * 64)
dense_skinny(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
             const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K) {
    using Op = DenseOp16<DT>;
    constexpr int STEP_BYTES = Op::KSTEP * Op::ELEM;   // 128
    __shared__ float red[kMaxWaves][AT][MT][4][64];
    const int WAVES = blockDim.x >> 6;   // 4, 8 or 16: the waves split K
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int n0 = blockIdx.x * 16 * AT;
    const int steps = (int)((K + Op::KSTEP - 1) / Op::KSTEP);   // the last step may be partial
    const int64_t row_bytes = K * Op::ELEM;
    const int o0 = 16 * kg, o1 = STEP_BYTES / 2 + 16 * kg;

    const Buf bufW(W, (uint32_t)N * (uint32_t)row_bytes);   // rows past N / M read as zeros
    const Buf bufX(X, (uint32_t)M * (uint32_t)row_bytes);
    uint32_t a_base[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
        a_base[t] = (uint32_t)(n0 + 16 * t + r) * (uint32_t)row_bytes;
    uint32_t b_base[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        b_base[mt] = (uint32_t)(mt * 16 + r) * (uint32_t)row_bytes;
    f32x4 acc[AT][MT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[t][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // contiguous K chunk per wave, K loop rotated per workgroup (as in the
    // sparse kernel)
    const int chunk = (steps + WAVES - 1) / WAVES;
    const int rot = (int)((blockIdx.x * 13u) % (unsigned)max(steps, 1));
    for (int i0 = 0; i0 < chunk; i0 += U) {
        uint4 a0[U][AT], a1[U][AT], b0[U][MT], b1[U][MT];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sl = wave * chunk + i0 + u;
            live[u] = i0 + u < chunk && sl < steps;
            int s = sl + rot;
            s = s >= steps ? s - steps : s;
            // 16-byte chunks past K (a partial last step) read as zeros
            const int64_t k0 = (int64_t)s * STEP_BYTES;
            const bool in0 = live[u] && k0 + o0 < row_bytes;
            const bool in1 = live[u] && k0 + o1 < row_bytes;
            const uint32_t d0 = in0 ? (uint32_t)(k0 + o0) : kOOB, d1 = in1 ? (uint32_t)(k0 + o1) : kOOB;
#pragma unroll
            for (int t = 0; t < AT; ++t) {
                a0[u][t] = bufW.ld16(a_base[t] + d0);
                a1[u][t] = bufW.ld16(a_base[t] + d1);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                b0[u][mt] = bufX.ld16(b_base[mt] + d0);
                b1[u][mt] = bufX.ld16(b_base[mt] + d1);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (live[u])
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int t = 0; t < AT; ++t)
                        acc[t][mt] = Op::mma(a0[u][t], a1[u][t], b0[u][mt], b1[u][mt], acc[t][mt]);
    }
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[wave][t][mt][i][lane] = acc[t][mt][i];
    __syncthreads();
    constexpr int TILE = 16 * 16 * MT;
    for (int o = threadIdx.x; o < AT * TILE; o += WAVES * 64) {
        const int t = o / TILE, ot = o - t * TILE;
        const int al = ot & 15, bl = ot >> 4;
        const int mt = bl >> 4, ln = ((al >> 2) << 4) | (bl & 15), i = al & 3;
        float v = 0.f;
        if constexpr (DT == SP24_I8) {
            // int32 partial sums (their bits in red): added exactly, converted once
            int vi = 0;
            for (int w = 0; w < WAVES; ++w)
                vi += __builtin_bit_cast(int, red[w][t][mt][i][ln]);
            v = (float)vi;
        } else {
            for (int w = 0; w < WAVES; ++w)   // fixed order: deterministic
                v += red[w][t][mt][i][ln];
        }
        const int n = n0 + 16 * t + al, m = bl;
        if (n < N && m < M) {
            if (sx)
                v *= sx[m];
            if (sw)
                v *= sw[n];
            store_out<OUT>(Y, (int64_t)m * N + n, v);
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// 5 to 16 rows of X: the construction of the sparse decode kernel for that
// range.  Waves split K into groups of 8 steps; W goes straight into
// registers; all 16 rows of X are staged in LDS, each row of a group one
// contiguous 1 KiB load with its 16-byte chunks XOR-permuted by the row
// number (16 rows read by one fragment load fall in 16 bank groups); AT
// 16-row tiles of W per workgroup; WV waves; the staging area then holds the
// cross-wave reduction.
template <sp24_dtype DT, sp24_dtype OUT, int AT, int WV>
__global__ void __launch_bounds__(WV * 64)
dense_skinny_x16(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
                 const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K) {
    using Op = DenseOp16<DT>;
    constexpr int STEP_BYTES = Op::KSTEP * Op::ELEM;   // 128
    constexpr int G = 8;                               // K steps per load group
    constexpr int X_ROW = G * STEP_BYTES;              // one row of X per group
    static_assert(X_ROW == 1024, "one 1 KiB load per staged row and group");
    constexpr int PER_WAVE = 16 * X_ROW;
    static_assert(AT * 4 * 64 * 4 <= PER_WAVE, "the reduction fits in the staging area");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[WV * PER_WAVE];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int n0 = blockIdx.x * 16 * AT;
    const int steps = (int)((K + Op::KSTEP - 1) / Op::KSTEP);   // the last step may be partial
    const int groups = (steps + G - 1) / G;
    const uint32_t row_bytes = (uint32_t)(K * Op::ELEM);
    const int o0 = 16 * kg, o1 = STEP_BYTES / 2 + 16 * kg;
    const Buf bufW(W, (uint32_t)N * row_bytes);   // rows past N / M read as zeros
    const Buf bufX(X, (uint32_t)M * row_bytes);
    uint8_t* my_x = lds + wave * PER_WAVE;
    const uint8_t* xr = my_x + X_ROW * r;
    uint32_t a_base[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
        a_base[t] = (uint32_t)(n0 + 16 * t + r) * row_bytes;
    f32x4 acc[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
        acc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int per_wave = (groups + WV - 1) / WV;
    const int rot = (int)((blockIdx.x * 5u) % (unsigned)max(groups, 1));
    for (int gi = 0; gi < per_wave; ++gi) {
        const int gl = wave * per_wave + gi;
        if (gl >= groups)
            break;
        const int g = gl + rot >= groups ? gl + rot - groups : gl + rot;
        const uint32_t k_first = (uint32_t)g * X_ROW;   // the group's first byte in a row
        // W: 16-byte chunks past K (a partial last step, or steps past it) read as zeros
        uint4 a0[AT][G], a1[AT][G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const uint32_t k0 = k_first + (uint32_t)u * STEP_BYTES;
            const bool in0 = k0 + o0 < row_bytes, in1 = k0 + o1 < row_bytes;
#pragma unroll
            for (int t = 0; t < AT; ++t) {
                a0[t][u] = bufW.ld16(in0 ? a_base[t] + k0 + o0 : kOOB);
                a1[t][u] = bufW.ld16(in1 ? a_base[t] + k0 + o1 : kOOB);
            }
        }
        // X row j: lane l fetches the chunk that belongs in slot l, chunk l ^ j
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t col = k_first + 16 * (lane ^ j);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bufX.r, (lds_void*)(my_x + X_ROW * j), 16,
                                                     (int)(col < row_bytes ? (uint32_t)j * row_bytes + col : kOOB),
                                                     0, 0, 0);
        }
        // this wave's loads have landed
        __builtin_amdgcn_s_waitcnt((0) | (0x7 << 4) | (0xF << 8));
        // steps past the end of K run on zeros and add nothing
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const uint4 b0 = *reinterpret_cast<const uint4*>(xr + 16 * ((8 * u + o0 / 16) ^ r));
            const uint4 b1 = *reinterpret_cast<const uint4*>(xr + 16 * ((8 * u + o1 / 16) ^ r));
#pragma unroll
            for (int t = 0; t < AT; ++t)
                acc[t] = Op::mma(a0[t][u], a1[t][u], b0, b1, acc[t]);
        }
        // the next group's loads reuse this wave's LDS: finish reading it
        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
    }

    // every wave is past its staging area before it holds the partial tiles
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);   // [WV][AT][4][64]
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[((wave * AT + t) * 4 + i) * 64 + lane] = acc[t][i];
    __syncthreads();
    for (int o = threadIdx.x; o < AT * 256; o += WV * 64) {
        const int t = o >> 8, ot = o & 255;
        const int al = ot & 15, bl = ot >> 4;
        const int ln = ((al >> 2) << 4) | bl, i = al & 3;
        float v = 0.f;
        if constexpr (DT == SP24_I8) {
            int vi = 0;
            for (int w = 0; w < WV; ++w)
                vi += __builtin_bit_cast(int, red[((w * AT + t) * 4 + i) * 64 + ln]);
            v = (float)vi;
        } else {
            for (int w = 0; w < WV; ++w)   // fixed order: deterministic
                v += red[((w * AT + t) * 4 + i) * 64 + ln];
        }
        const int n = n0 + 16 * t + al, m = bl;
        if (n < N && m < M) {
            if (sx)
                v *= sx[m];
            if (sw)
                v *= sw[n];
            store_out<OUT>(Y, (int64_t)m * N + n, v);
        }
    }
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t dispatch(const DenseArgs& g, hipStream_t s, const char** kname) {
    const int N = (int)g.N, M = (int)g.M;
    const uint8_t* W = (const uint8_t*)g.W;
    const uint8_t* X = (const uint8_t*)g.X;
    // the same split as the sparse dispatch: few rows of X on a narrow output
    // go to the K-splitting decode kernel, everything else to the tile kernels
    if (M <= 16 || (M <= 64 && (N + 127) / 128 < 128)) {
        const int tiles16 = (N + 15) / 16;
        const int steps = (int)((g.K + DenseOp16<DT>::KSTEP - 1) / DenseOp16<DT>::KSTEP);
        const int mt = (M + 15) / 16;
        const bool a32 = mt >= 2 && tiles16 / 2 >= 160;
        const int64_t wgs = a32 ? (tiles16 + 1) / 2 : tiles16;
        int waves = 16;
        while (waves > 4 && (wgs * waves > 8192 || steps < waves * 2))
            waves >>= 1;
#define DENSE_SKINNY(MT, U, AT, NAME)                                                                \
    do {                                                                                             \
        if (!g.dry)                                                                                  \
            hipLaunchKernelGGL((dense_skinny<DT, OUT, MT, U, AT>), dim3((N + 16 * AT - 1) / (16 * AT)),  \
                               dim3(waves * 64), 0, s, W, X, g.scale_x, g.scale_w, g.Y, N, M, g.K);  \
        if (kname) *kname = NAME;                                                                    \
    } while (0)
        // 17 to 64 rows of X: 32-row W tiles when that still leaves 160 or more
        // workgroups (each X fragment then serves two W tiles), as the sparse
        // decode kernel does
        // 5 to 16 rows: staged in LDS, with the sparse decode kernel's choice
        // of waves and of 32-row W tiles
        if (mt <= 1 && M > 4) {
            const int groups = (steps + 7) / 8;
            int wv = 8;
            while (wv > 2 && groups < wv)
                wv >>= 1;
            const bool at2 = tiles16 / 2 >= 192;
            if (at2 && tiles16 / 2 >= 3 * 256)
                wv = min(wv, 4);
#define DENSE_X16(AT, NAME)                                                                          \
    do {                                                                                             \
        const dim3 grid((N + 16 * AT - 1) / (16 * AT));                                              \
        if (!g.dry) {                                                                                \
            if (wv <= 4)                                                                             \
                hipLaunchKernelGGL((dense_skinny_x16<DT, OUT, AT, 4>), grid, dim3(256), 0, s, W, X,  \
                                   g.scale_x, g.scale_w, g.Y, N, M, g.K);                            \
            else                                                                                     \
                hipLaunchKernelGGL((dense_skinny_x16<DT, OUT, AT, 8>), grid, dim3(512), 0, s, W, X,  \
                                   g.scale_x, g.scale_w, g.Y, N, M, g.K);                            \
        }                                                                                            \
        if (kname) *kname = NAME;                                                                    \
    } while (0)
            if (at2) DENSE_X16(2, "dense_skinny_m16_a32");
            else DENSE_X16(1, "dense_skinny_m16");
#undef DENSE_X16
        }
        else if (mt <= 1) DENSE_SKINNY(1, 4, 1, "dense_skinny_m1");
        else if (mt == 2 && a32) DENSE_SKINNY(2, 2, 2, "dense_skinny_m2_a32");
        else if (mt == 2) DENSE_SKINNY(2, 2, 1, "dense_skinny_m2");
        else if (a32) DENSE_SKINNY(4, 2, 2, "dense_skinny_m4_a32");
        else DENSE_SKINNY(4, 2, 1, "dense_skinny_m4");
#undef DENSE_SKINNY
    } else {
        return launch_dense_gemm_big(g, s, kname);
    }
    return g.dry ? hipSuccess : hipGetLastError();
}

}  // namespace

hipError_t launch_dense_gemm(const DenseArgs& g, hipStream_t s, const char** kname) {
    if (g.M == 0 || g.N == 0)
        return hipSuccess;
    switch (g.in_dt) {
    case SP24_BF16:
        if (g.out_dt == SP24_BF16) return dispatch<SP24_BF16, SP24_BF16>(g, s, kname);
        if (g.out_dt == SP24_F16) return dispatch<SP24_BF16, SP24_F16>(g, s, kname);
        return dispatch<SP24_BF16, SP24_F32>(g, s, kname);
    case SP24_F16:
        if (g.out_dt == SP24_F16) return dispatch<SP24_F16, SP24_F16>(g, s, kname);
        if (g.out_dt == SP24_BF16) return dispatch<SP24_F16, SP24_BF16>(g, s, kname);
        return dispatch<SP24_F16, SP24_F32>(g, s, kname);
    case SP24_E4M3:
        if (g.out_dt == SP24_BF16) return dispatch<SP24_E4M3, SP24_BF16>(g, s, kname);
        return dispatch<SP24_E4M3, SP24_F32>(g, s, kname);
    case SP24_I8:
        if (g.out_dt == SP24_BF16) return dispatch<SP24_I8, SP24_BF16>(g, s, kname);
        return dispatch<SP24_I8, SP24_F32>(g, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
