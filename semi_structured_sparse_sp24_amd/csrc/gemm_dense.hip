// gemm_dense.hip -- dense GEMM baseline Y = X * W^T on gfx950 MFMA.
//
// The baseline every sparse tactic is timed against and the target of every
// fallback ("Production 2:4 Structured Sparsity for LLMs", sections "Sparse
// Tactic Audit" and "Dense Fallback and Hybrid Sparsity Design").  It has
// the same two shapes as the sparse kernels so that the comparison is
// between kernels of the same construction:
//   skinny  M <= 64: the workgroup owns 16 rows of W and all of X; waves
//           split K; v_mfma_f32_16x16x32 (16-bit, two per 64-K step) or
//           v_mfma_scale_f32_16x16x128_f8f6f4 (fp8, unit scales).
//   tiled   128 x 128 tile, double-buffered LDS, 2 x 2 waves each owning
//           2 x 2 fragments of v_mfma_f32_32x32x16 (16-bit) or
//           v_mfma_scale_f32_32x32x64_f8f6f4 (fp8).
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
template <>
struct DenseOp16<SP24_E4M3> {
    static constexpr int KSTEP = 128, ELEM = 1;
    __device__ static __forceinline__ f32x4 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x4 c) {
        struct { uint4 x, y; } aa = {a0, a1}, bb = {b0, b1};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            __builtin_bit_cast(i32x8, aa), __builtin_bit_cast(i32x8, bb), c, 0, 0, 0, 0x7f, 0, 0x7f);
    }
};

// 32x32 output fragment over one 16-byte-per-lane K slice (16-bit: 16 K
// with 8 per lane; fp8: 64 K with 32 bytes per lane = two slices).
template <sp24_dtype DT>
struct DenseOp32;
template <>
struct DenseOp32<SP24_BF16> {
    static constexpr int KSTEP = 64, ELEM = 2, SUB = 4;   // 4 instructions per 64-K step
    static constexpr int SUB_BYTES = 32;                  // bytes of K per instruction per row
    __device__ static __forceinline__ f32x16 mma(uint4 a0, uint4, uint4 b0, uint4, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                       __builtin_bit_cast(bf16x8, b0), c, 0, 0, 0);
    }
};
template <>
struct DenseOp32<SP24_F16> {
    static constexpr int KSTEP = 64, ELEM = 2, SUB = 4;
    static constexpr int SUB_BYTES = 32;
    __device__ static __forceinline__ f32x16 mma(uint4 a0, uint4, uint4 b0, uint4, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a0),
                                                      __builtin_bit_cast(f16x8, b0), c, 0, 0, 0);
    }
};
template <>
struct DenseOp32<SP24_E4M3> {
    static constexpr int KSTEP = 128, ELEM = 1, SUB = 2;  // 2 instructions per 128-K step
    static constexpr int SUB_BYTES = 64;
    __device__ static __forceinline__ f32x16 mma(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x16 c) {
        struct { uint4 x, y; } aa = {a0, a1}, bb = {b0, b1};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_bit_cast(i32x8, aa), __builtin_bit_cast(i32x8, bb), c, 0, 0, 0, 0x7f, 0, 0x7f);
    }
};

// ------------------------------------------------------------------ skinny
constexpr int kMaxWaves = 16;

template <sp24_dtype DT, sp24_dtype OUT, int MT, int U>
__global__ void __launch_bounds__(kMaxWaves * 64)
dense_skinny(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
             const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K) {
    using Op = DenseOp16<DT>;
    constexpr int STEP_BYTES = Op::KSTEP * Op::ELEM;   // 128
    __shared__ float red[kMaxWaves][MT][4][64];
    const int WAVES = blockDim.x >> 6;   // 4, 8 or 16: the waves split K
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int steps = (int)((K + Op::KSTEP - 1) / Op::KSTEP);   // the last step may be partial
    const int64_t row_bytes = K * Op::ELEM;
    const int o0 = 16 * kg, o1 = STEP_BYTES / 2 + 16 * kg;

    const Buf bufW(W, (uint32_t)N * (uint32_t)row_bytes);   // rows past N / M read as zeros
    const Buf bufX(X, (uint32_t)M * (uint32_t)row_bytes);
    const uint32_t a_base = (uint32_t)(n0 + r) * (uint32_t)row_bytes;
    uint32_t b_base[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        b_base[mt] = (uint32_t)(mt * 16 + r) * (uint32_t)row_bytes;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // contiguous K chunk per wave, K loop rotated per workgroup (as in the
    // sparse kernel)
    const int chunk = (steps + WAVES - 1) / WAVES;
    const int rot = (int)((blockIdx.x * 13u) % (unsigned)max(steps, 1));
    for (int i0 = 0; i0 < chunk; i0 += U) {
        uint4 a0[U], a1[U], b0[U][MT], b1[U][MT];
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
            a0[u] = bufW.ld16(a_base + d0);
            a1[u] = bufW.ld16(a_base + d1);
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
                    acc[mt] = Op::mma(a0[u], a1[u], b0[u][mt], b1[u][mt], acc[mt]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[wave][mt][i][lane] = acc[mt][i];
    __syncthreads();
    for (int o = threadIdx.x; o < 16 * 16 * MT; o += WAVES * 64) {
        const int al = o & 15, bl = o >> 4;
        const int mt = bl >> 4, ln = ((al >> 2) << 4) | (bl & 15), i = al & 3;
        float v = 0.f;
        for (int w = 0; w < WAVES; ++w)   // fixed order: deterministic
            v += red[w][mt][i][ln];
        const int n = n0 + al, m = bl;
        if (n < N && m < M) {
            if (sx)
                v *= sx[m];
            if (sw)
                v *= sw[n];
            store_out<OUT>(Y, (int64_t)m * N + n, v);
        }
    }
}

// ------------------------------------------------------------------ tiled
template <sp24_dtype DT, sp24_dtype OUT, int FA, int FB>
__global__ void __launch_bounds__(256)
dense_tiled(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
            const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K, int tiles_n) {
    using Op = DenseOp32<DT>;
    constexpr int BA = 2 * FA * 32, BB = 2 * FB * 32;
    constexpr int STEP_BYTES = Op::KSTEP * Op::ELEM;     // 128
    constexpr int STRIDE = STEP_BYTES + 16;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BA * STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BB * STRIDE];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 31, kg = lane >> 5;
    const int wa = wave >> 1, wb = wave & 1;
    const int ta = blockIdx.x % tiles_n, tb = blockIdx.x / tiles_n;
    const int a0 = ta * BA, b0 = tb * BB;
    const int steps = (int)((K + Op::KSTEP - 1) / Op::KSTEP);   // the last step may be partial
    const int64_t row_bytes = K * Op::ELEM;

    constexpr int A_CHUNKS = BA * 8 / 256, B_CHUNKS = BB * 8 / 256;
    const int chunk_col = (tid & 7) * 16;   // byte column of this thread's chunks in a step
    const Buf bufW(W, (uint32_t)N * (uint32_t)row_bytes);   // rows past N / M read as zeros
    const Buf bufX(X, (uint32_t)M * (uint32_t)row_bytes);
    uint32_t ga[A_CHUNKS];
    int la[A_CHUNKS];
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
        int c = tid + j * 256, row = c >> 3, col = c & 7;
        ga[j] = (uint32_t)(a0 + row) * (uint32_t)row_bytes + col * 16;
        la[j] = row * STRIDE + col * 16;
    }
    uint32_t gb[B_CHUNKS];
    int lb[B_CHUNKS];
#pragma unroll
    for (int j = 0; j < B_CHUNKS; ++j) {
        int c = tid + j * 256, row = c >> 3, col = c & 7;
        gb[j] = (uint32_t)(b0 + row) * (uint32_t)row_bytes + col * 16;
        lb[j] = row * STRIDE + col * 16;
    }
    const uint4 zero = make_uint4(0, 0, 0, 0);
    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    // K loop rotated per workgroup (as in the sparse kernel)
    const int rot = (int)((blockIdx.x * 13u) % (unsigned)steps);
    auto gload = [&](int sl) {
        const int s = sl + rot >= steps ? sl + rot - steps : sl + rot;
        // a 16-byte chunk past K (a partial last step) reads as zeros
        const bool in = (int64_t)s * STEP_BYTES + chunk_col < row_bytes;
        const uint32_t ks = in ? (uint32_t)s * STEP_BYTES : kOOB;
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j)
            ra[j] = bufW.ld16(ga[j] + ks);
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j)
            rb[j] = bufX.ld16(gb[j] + ks);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j)
            *reinterpret_cast<uint4*>(&lds_a[buf][la[j]]) = ra[j];
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j)
            *reinterpret_cast<uint4*>(&lds_b[buf][lb[j]]) = rb[j];
    };

    f32x16 acc[FA][FB];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
            acc[i][j] = (f32x16){};

    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        if (s + 1 < steps)
            gload(s + 1);
#pragma unroll
        for (int q = 0; q < Op::SUB; ++q) {
            // 16-bit: this lane's 16 B at q*32 + 16*kg; fp8: 32 B at q*64 + 32*kg
            const int off0 = q * Op::SUB_BYTES + (Op::ELEM == 2 ? 16 * kg : 32 * kg);
            const int off1 = off0 + 16;
            uint4 fa0[FA], fa1[FA];
#pragma unroll
            for (int i = 0; i < FA; ++i) {
                const uint8_t* p = &lds_a[buf][(wa * FA * 32 + i * 32 + r) * STRIDE];
                fa0[i] = *reinterpret_cast<const uint4*>(p + off0);
                if (Op::ELEM == 1)
                    fa1[i] = *reinterpret_cast<const uint4*>(p + off1);
                else
                    fa1[i] = zero;
            }
#pragma unroll
            for (int j = 0; j < FB; ++j) {
                const uint8_t* p = &lds_b[buf][(wb * FB * 32 + j * 32 + r) * STRIDE];
                uint4 fb0 = *reinterpret_cast<const uint4*>(p + off0);
                uint4 fb1 = Op::ELEM == 1 ? *reinterpret_cast<const uint4*>(p + off1) : zero;
#pragma unroll
                for (int i = 0; i < FA; ++i)
                    acc[i][j] = Op::mma(fa0[i], fa1[i], fb0, fb1, acc[i][j]);
            }
        }
        if (s + 1 < steps)
            lstore(buf ^ 1);
        __syncthreads();
    }

    // D[8*(q/4) + 4*kg + q%4][r] of fragment (i, j): a = W row, b = X row
#pragma unroll
    for (int i = 0; i < FA; ++i) {
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int m = b0 + wb * FB * 32 + j * 32 + r;
            if (m >= M)
                continue;
            const float fsx = sx ? sx[m] : 1.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int n = a0 + wa * FA * 32 + i * 32 + 8 * h + 4 * kg;
                f32x4 v;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[q] = acc[i][j][4 * h + q] * fsx * (sw && n + q < N ? sw[n + q] : 1.f);
                const int64_t off = (int64_t)m * N + n;
                if (n + 3 < N && (off & 3) == 0) {
                    store_out4<OUT>(Y, off, v);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < N)
                            store_out<OUT>(Y, off + q, v[q]);
                }
            }
        }
    }
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t dispatch(const DenseArgs& g, hipStream_t s, const char** kname) {
    const int N = (int)g.N, M = (int)g.M;
    const uint8_t* W = (const uint8_t*)g.W;
    const uint8_t* X = (const uint8_t*)g.X;
    if (M <= 64) {
        const int tiles16 = (N + 15) / 16;
        const int steps = (int)((g.K + DenseOp16<DT>::KSTEP - 1) / DenseOp16<DT>::KSTEP);
        int waves = 16;
        while (waves > 4 && ((int64_t)tiles16 * waves > 8192 || steps < waves * 2))
            waves >>= 1;
#define DENSE_SKINNY(MT, U)                                                                          \
    do {                                                                                             \
        if (!g.dry)                                                                                  \
            hipLaunchKernelGGL((dense_skinny<DT, OUT, MT, U>), dim3(tiles16), dim3(waves * 64), 0, s,  \
                               W, X, g.scale_x, g.scale_w, g.Y, N, M, g.K);                          \
        if (kname) *kname = "dense_skinny_m" #MT;                                                    \
    } while (0)
        const int mt = (M + 15) / 16;
        if (mt <= 1) DENSE_SKINNY(1, 4);
        else if (mt == 2) DENSE_SKINNY(2, 2);
        else DENSE_SKINNY(4, 2);
#undef DENSE_SKINNY
    } else if ((int64_t)((N + 255) / 256) * ((M + 255) / 256) >= 192) {
        return launch_dense_gemm_big(g, s, kname);
    } else {
        constexpr int FA = 2, FB = 2, BA = 2 * FA * 32, BB = 2 * FB * 32;
        const int tiles_n = (N + BA - 1) / BA, tiles_m = (M + BB - 1) / BB;
        if (!g.dry)
            hipLaunchKernelGGL((dense_tiled<DT, OUT, FA, FB>), dim3(tiles_n * tiles_m), dim3(256), 0, s, W,
                               X, g.scale_x, g.scale_w, g.Y, N, M, g.K, tiles_n);
        if (kname) *kname = "dense_tiled_128x128";
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
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
