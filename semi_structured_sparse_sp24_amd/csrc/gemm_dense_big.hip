// gemm_dense_big.hip -- dense GEMM baseline Y = X * W^T for more than 16
// rows of X, built the same way as the sparse tile kernels (same tile shapes
// and tile choice) so that the tactic comparison is between kernels of the
// same construction ("Production 2:4 Structured Sparsity for LLMs", section
// "Sparse Tactic Audit").  Shown for the 256 x 256 tile:
//
//   - tile 256 (W rows) x 256 (X rows); 8 waves in a 4 x 2 grid (two per
//     SIMD), each owning 64 x 128 = 2 x 4 fragments of v_mfma_f32_32x32x16
//     (16-bit) or v_mfma_scale_f32_32x32x64_f8f6f4 (fp8, unit scales);
//   - one stage = one 128-byte slice of every row of both operands (64 K for
//     16-bit, 128 K for fp8): 64 KB; two stages in LDS, filled by direct
//     global->LDS loads while the other is consumed;
//   - 16-byte chunks XOR-swizzled by row for conflict-free fragment reads;
//   - XCD-aware grouped tile order, K start rotated per group.
// Any K with whole 16-byte row chunks is accepted: chunks past the end of a
// row read as zeros.
#include "mfma_ops.h"

namespace sp24 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// Tile shapes: BA rows of W x BB rows of X, WA x WB waves, OCC workgroups per CU.
template <int BA_, int BB_, int WA_, int WB_, int OCC_>
struct DTile {
    static constexpr int BA = BA_, BB = BB_, WA = WA_, WB = WB_, OCC = OCC_;
    static constexpr int WAVES = WA * WB, THREADS = 64 * WAVES;
    static constexpr int FA = BA / 32 / WA, FB = BB / 32 / WB;    // 32x32 fragments per wave
    static constexpr int LA = BA * 128 / 1024 / WAVES;            // 1 KiB loads of W per wave and stage
    static constexpr int LB = BB * 128 / 1024 / WAVES;            // ... of X
};
using D256x256 = DTile<256, 256, 4, 2, 1>;
using D256x128 = DTile<256, 128, 4, 2, 1>;
using D128x128 = DTile<128, 128, 2, 4, 2>;
using D256x64 = DTile<256, 64, 4, 2, 1>;
using D128x64 = DTile<128, 64, 4, 2, 2>;

template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

template <sp24_dtype DT>
struct Dense32;
template <>
struct Dense32<SP24_BF16> {
    static constexpr int KSTEP = 64, SUB = 4, CHUNKS = 1;   // per instruction: 1 chunk of 16 B per lane
    __device__ static __forceinline__ f32x16 mma(const uint4* a, const uint4* b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                       __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
    }
};
template <>
struct Dense32<SP24_F16> {
    static constexpr int KSTEP = 64, SUB = 4, CHUNKS = 1;
    __device__ static __forceinline__ f32x16 mma(const uint4* a, const uint4* b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                                      __builtin_bit_cast(f16x8, b[0]), c, 0, 0, 0);
    }
};
// int8: 32 K (32 bytes per row) per instruction, int32 accumulation in the
// accumulator registers' bits, converted in the epilogue.
template <>
struct Dense32<SP24_I8> {
    static constexpr int KSTEP = 128, SUB = 4, CHUNKS = 1;
    __device__ static __forceinline__ f32x16 mma(const uint4* a, const uint4* b, f32x16 c) {
        typedef __attribute__((ext_vector_type(16))) int i32x16;
        return __builtin_bit_cast(f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(
            __builtin_bit_cast(i32x4, a[0]), __builtin_bit_cast(i32x4, b[0]), __builtin_bit_cast(i32x16, c), 0, 0, 0));
    }
};
template <>
struct Dense32<SP24_E4M3> {
    static constexpr int KSTEP = 128, SUB = 2, CHUNKS = 2;  // 32 B per lane per instruction
    __device__ static __forceinline__ f32x16 mma(const uint4* a, const uint4* b, f32x16 c) {
        struct { uint4 x, y; } aa = {a[0], a[1]}, bb = {b[0], b[1]};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            __builtin_bit_cast(i32x8, aa), __builtin_bit_cast(i32x8, bb), c, 0, 0, 0, 0x7f, 0, 0x7f);
    }
};

// Workgroup b of nwg -> its place in an XCD-aware order (consecutive places
// run on one XCD), and place t -> (group, W tile, X tile) in groups of 8 W
// tiles x all X tiles.
__device__ __forceinline__ int dxcd_order(int b, int nwg) {
    const int xcd = b & 7, local = b >> 3;
    const int per_xcd = (nwg + 7) >> 3, full = nwg & 7 ? (nwg & 7) : 8;
    return xcd < full ? xcd * per_xcd + local : full * per_xcd + (xcd - full) * (per_xcd - 1) + local;
}
struct DTilePos {
    int group, ta, tb;
};
__device__ __forceinline__ DTilePos dtile_pos(int t, int tiles_a, int tiles_b) {
    constexpr int G = 8;
    const int group = t / (G * tiles_b), within = t - group * G * tiles_b;
    const int g_rows = min(G, tiles_a - group * G);
    return {group, group * G + within % g_rows, within / g_rows};
}

// One output tile: W rows [a0, a0 + TL::BA) x X rows [b0, b0 + TL::BB), over
// the whole K, in two LDS stages per operand (a0s/a1s, b0s/b1s).
template <sp24_dtype DT, sp24_dtype OUT, class TL>
__device__ __forceinline__ void dense_tile(uint8_t* a0s, uint8_t* a1s, uint8_t* b0s, uint8_t* b1s,
                                           const uint8_t* __restrict__ W, const uint8_t* __restrict__ X,
                                           const float* __restrict__ sx, const float* __restrict__ sw,
                                           void* __restrict__ Y, int N, int M, int64_t K, int a0, int b0,
                                           int group) {
    using Op = Dense32<DT>;
    constexpr int kBA = TL::BA, kBB = TL::BB, kWB = TL::WB, kFA = TL::FA, kFB = TL::FB;
    constexpr int LA = TL::LA, LB = TL::LB;
    static_assert(LA * TL::WAVES * 1024 == kBA * 128 && LB * TL::WAVES * 1024 == kBB * 128, "whole loads");
    constexpr int LOADS = LA + LB;                  // per wave per stage

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, kg = lane >> 5;
    const int wa = wave / kWB, wb = wave % kWB;

    const uint32_t row_bytes = (uint32_t)K * (DT == SP24_E4M3 || DT == SP24_I8 ? 1 : 2);
    const int steps = (int)((row_bytes + 127) / 128);   // the last may be partial
    const Buf bufW(W, (uint32_t)N * row_bytes);           // rows past N / M read as zeros
    const Buf bufX(X, (uint32_t)M * row_bytes);

    // ---- this wave's loads: LA x 1 KiB of W rows and LB of X rows per stage
    // (8 rows per load; lane l fetches the chunk that the row's XOR swizzle
    // puts in slot l & 7)
    uint32_t ga[LA], gb[LB];
    int ca[LA], cb[LB];   // byte column of the chunk each lane fetches (for the partial last step)
#pragma unroll
    for (int j = 0; j < LA; ++j) {
        const int row = 8 * (LA * wave + j) + (lane >> 3);
        ca[j] = 16 * ((lane & 7) ^ ((row >> 1) & 7));
        ga[j] = (uint32_t)(a0 + row) * row_bytes + ca[j];
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        const int row = 8 * (LB * wave + j) + (lane >> 3);
        cb[j] = 16 * ((lane & 7) ^ ((row >> 1) & 7));
        gb[j] = (uint32_t)(b0 + row) * row_bytes + cb[j];
    }
    const int rot = (int)(((unsigned)group * 13u) % (unsigned)steps);
    // The step's byte offset goes in the (uniform) scalar offset, kOOB for the
    // padded steps past the end.  A lane whose chunk lies past the end of its
    // row (the partial last step) moves its vector offset to kOOB instead,
    // which with any scalar offset of a row is past the operand's size
    // (< 2 GiB), so it reads zeros.  Both offsets are never kOOB at once (their
    // sum would wrap).
    auto issue = [&](uint8_t* as, uint8_t* bs, int sl) {
        int s = sl + rot;
        s = s >= steps ? s - steps : s;
        const bool live = sl < steps;
        const uint32_t so = live ? (uint32_t)s * 128 : kOOB;
#pragma unroll
        for (int j = 0; j < LA; ++j)
            dma16_lds(bufW, as + 1024 * (LA * wave + j), !live || so + ca[j] < row_bytes ? ga[j] : kOOB, so);
#pragma unroll
        for (int j = 0; j < LB; ++j)
            dma16_lds(bufX, bs + 1024 * (LB * wave + j), !live || so + cb[j] < row_bytes ? gb[j] : kOOB, so);
    };

    f32x16 acc[kFA][kFB];
#pragma unroll
    for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int j = 0; j < kFB; ++j)
            acc[i][j] = (f32x16){};

    const int swz = (r >> 1) & 7;
    auto compute = [&](const uint8_t* as, const uint8_t* bs) {
#pragma unroll
        for (int q = 0; q < Op::SUB; ++q) {
            uint4 fa[kFA][Op::CHUNKS], fb[kFB][Op::CHUNKS];
#pragma unroll
            for (int h = 0; h < Op::CHUNKS; ++h) {
                // chunk of K this lane supplies: 16-bit 2q + kg; fp8 4q + 2kg + h
                const int c = Op::CHUNKS == 1 ? 2 * q + kg : 4 * q + 2 * kg + h;
                const int off = 16 * (c ^ swz);
#pragma unroll
                for (int i = 0; i < kFA; ++i)
                    fa[i][h] = *reinterpret_cast<const uint4*>(as + (wa * 32 * kFA + i * 32 + r) * 128 + off);
#pragma unroll
                for (int j = 0; j < kFB; ++j)
                    fb[j][h] = *reinterpret_cast<const uint4*>(bs + (wb * 32 * kFB + j * 32 + r) * 128 + off);
            }
#pragma unroll
            for (int i = 0; i < kFA; ++i)
#pragma unroll
                for (int j = 0; j < kFB; ++j)
                    acc[i][j] = Op::mma(fa[i], fb[j], acc[i][j]);
        }
    };

    // ---- two stages: the loads of step s+1 land while step s is consumed;
    // the step count is padded to even (padded steps read zeros)
    issue(a0s, b0s, 0);
    const int steps2 = (steps + 1) / 2 * 2;
    for (int s = 0; s < steps2; s += 2) {
        wait_vmcnt_lgkm0<0>();
        barrier_lds();
        issue(a1s, b1s, s + 1);
        compute(a0s, b0s);
        wait_vmcnt_lgkm0<0>();
        barrier_lds();
        issue(a0s, b0s, s + 2);
        compute(a1s, b1s);
    }
    wait_vmcnt_lgkm0<0>();

    // ---- epilogue: D[8*(v/4) + 4*kg + v%4][r] of fragment (i, j); a = W row (n), b = X row (m)
    auto value = [&](const f32x16& accf, int h, int n, float fsx) {
        f32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] = accf[4 * h + q] * fsx * (sw && n + q < N ? sw[n + q] : 1.f);
        return v;
    };
    if constexpr (OUT != SP24_F32) {
        // Y is X-row-major, so a lane's four consecutive outputs are 8 bytes
        // of one row of Y and a store instruction writes 16-byte pieces of 32
        // rows.  As in the sparse tile kernels, a whole block of the wave (EA
        // rows of W x EB rows of X) is staged in the free stage memory, row m
        // of Y as a run of EA outputs with its 16-byte chunks XOR-permuted by
        // m, and written back as whole 16-byte pieces, CPR lanes per row, by
        // streaming (non-temporal) stores.
        constexpr int EA = 32 * kFA, EB = 32 * kFB;
        constexpr int W_STG = EA * EB * 2;                    // staging bytes per wave
        constexpr int PA = kBA * 128 / W_STG, PB = kBB * 128 / W_STG;   // waves per W / X stage
        static_assert(2 * PA + 2 * PB >= TL::WAVES, "staging fits the stages");
        constexpr int CPR = EA / 8;                           // 16-byte chunks per staged row
        constexpr int CPP = 64 / CPR;                         // rows per wave-wide read
        static_assert(CPR >= 4 && CPR <= 16 && EB % CPP == 0, "staged block shape");
        const int n_w = a0 + wa * EA, m_w = b0 + wb * EB;
        if ((N & 7) == 0 && ((uintptr_t)Y & 15) == 0) {
            // every wave is done with the stages
            __syncthreads();
            if (n_w + EA <= N && m_w + EB <= M) {
                const int w = wave;
                uint8_t* stg = w < PA ? a0s + w * W_STG
                             : w < 2 * PA ? a1s + (w - PA) * W_STG
                             : w < 2 * PA + PB ? b0s + (w - 2 * PA) * W_STG
                                               : b1s + (w - 2 * PA - PB) * W_STG;
                auto slot = [](int ml, int c) { return 16 * (c ^ ((ml / (16 / CPR)) & (CPR - 1))); };
#pragma unroll
                for (int i = 0; i < kFA; ++i) {
#pragma unroll
                    for (int j = 0; j < kFB; ++j) {
                        const int ml = j * 32 + r;
                        const float fsx = sx ? sx[m_w + ml] : 1.f;
                        const f32x16 accf = acc_to_f32<DT>(acc[i][j]);
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            const int nl = i * 32 + 8 * h + 4 * kg;
                            const f32x4 v = value(accf, h, n_w + nl, fsx);
                            uint16_t hv[4];
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                hv[q] = OUT == SP24_BF16 ? f32_to_bf16_rne(v[q]) : f32_to_f16_rne(v[q]);
                            *reinterpret_cast<uint2*>(stg + ml * (EA * 2) + slot(ml, nl >> 3) + 8 * ((nl >> 2) & 1)) =
                                make_uint2(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16));
                        }
                    }
                }
                // this wave's LDS writes complete before it reads them back
                __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
                __builtin_amdgcn_wave_barrier();
                uint16_t* const y = reinterpret_cast<uint16_t*>(Y);
#pragma unroll
                for (int pass = 0; pass < EB / CPP; ++pass) {
                    const int ml = pass * CPP + lane / CPR, c = lane % CPR;
                    const uint4 d = *reinterpret_cast<const uint4*>(stg + ml * (EA * 2) + slot(ml, c));
                    store_stream(y + (int64_t)(m_w + ml) * N + n_w + 8 * c, d);
                }
                return;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int j = 0; j < kFB; ++j) {
            const int m = b0 + wb * 32 * kFB + j * 32 + r;
            if (m >= M)
                continue;
            const float fsx = sx ? sx[m] : 1.f;
            const f32x16 accf = acc_to_f32<DT>(acc[i][j]);
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const int n = a0 + wa * 32 * kFA + i * 32 + 8 * h + 4 * kg;
                if (n >= N)
                    continue;
                const f32x4 v = value(accf, h, n, fsx);
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

template <sp24_dtype DT, sp24_dtype OUT, class TL>
__global__ void __launch_bounds__(TL::THREADS, TL::OCC)
dense_big(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
          const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K, int tiles_a,
          int tiles_b) {
    __shared__ __attribute__((aligned(1024))) uint8_t a0s[TL::BA * 128], a1s[TL::BA * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t b0s[TL::BB * 128], b1s[TL::BB * 128];
    const DTilePos p = dtile_pos(dxcd_order((int)blockIdx.x, (int)gridDim.x), tiles_a, tiles_b);
    dense_tile<DT, OUT, TL>(a0s, a1s, b0s, b1s, W, X, sx, sw, Y, N, M, K, p.ta * TL::BA, p.tb * TL::BB, p.group);
}

// The 256 x 256 grid with a short last round, as the sparse tile kernels run
// it: the first n_big tiles (whole rounds) as 256 x 256, each later tile as
// `parts` smaller tiles (four 128 x 128 quarters, or two 256 x 128 halves),
// in the big tile's LDS.
template <sp24_dtype DT, sp24_dtype OUT>
__global__ void __launch_bounds__(D256x256::THREADS, 1)
dense_big_tail(const uint8_t* __restrict__ W, const uint8_t* __restrict__ X, const float* __restrict__ sx,
               const float* __restrict__ sw, void* __restrict__ Y, int N, int M, int64_t K, int tiles_a,
               int tiles_b, int n_big, int parts) {
    static_assert(D128x128::THREADS == D256x256::THREADS && D256x128::THREADS == D256x256::THREADS,
                  "one block size");
    __shared__ __attribute__((aligned(1024))) uint8_t a0s[256 * 128], a1s[256 * 128];
    __shared__ __attribute__((aligned(1024))) uint8_t b0s[256 * 128], b1s[256 * 128];
    const int b = (int)blockIdx.x;
    if (b < n_big) {
        const DTilePos p = dtile_pos(dxcd_order(b, n_big), tiles_a, tiles_b);
        dense_tile<DT, OUT, D256x256>(a0s, a1s, b0s, b1s, W, X, sx, sw, Y, N, M, K, p.ta * 256, p.tb * 256,
                                      p.group);
    } else if (parts == 2) {
        // n_big is a multiple of 8, so b - n_big keeps b's XCD
        const int q = dxcd_order(b - n_big, (int)gridDim.x - n_big);
        const DTilePos p = dtile_pos(n_big + q / 2, tiles_a, tiles_b);
        dense_tile<DT, OUT, D256x128>(a0s, a1s, b0s, b1s, W, X, sx, sw, Y, N, M, K, p.ta * 256,
                                      p.tb * 256 + 128 * (q & 1), p.group);
    } else {
        // n_big is a multiple of 8, so b - n_big keeps b's XCD
        const int q = dxcd_order(b - n_big, (int)gridDim.x - n_big);
        const DTilePos p = dtile_pos(n_big + q / 4, tiles_a, tiles_b);
        dense_tile<DT, OUT, D128x128>(a0s, a1s, b0s, b1s, W, X, sx, sw, Y, N, M, K,
                                      p.ta * 256 + 128 * ((q >> 1) & 1), p.tb * 256 + 128 * (q & 1), p.group);
    }
}

template <sp24_dtype DT, sp24_dtype OUT, class TL>
hipError_t launch_tile(const DenseArgs& g, hipStream_t s, const char** kname, const char* name) {
    const int N = (int)g.N, M = (int)g.M;
    const int tiles_a = (N + TL::BA - 1) / TL::BA, tiles_b = (M + TL::BB - 1) / TL::BB;
    if (kname)
        *kname = name;
    if (g.dry)
        return hipSuccess;
    hipLaunchKernelGGL((dense_big<DT, OUT, TL>), dim3(tiles_a * tiles_b), dim3(TL::THREADS), 0, s,
                       (const uint8_t*)g.W, (const uint8_t*)g.X, g.scale_x, g.scale_w, g.Y, N, M, g.K, tiles_a,
                       tiles_b);
    return hipGetLastError();
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_tail(const DenseArgs& g, hipStream_t s, const char** kname, int64_t n_big, int64_t n_split,
                       int parts) {
    const int N = (int)g.N, M = (int)g.M;
    const int tiles_a = (N + 255) / 256, tiles_b = (M + 255) / 256;
    if (kname)
        *kname = "dense_big_256x256_tail";
    if (g.dry)
        return hipSuccess;
    hipLaunchKernelGGL((dense_big_tail<DT, OUT>), dim3((unsigned)(n_big + parts * n_split)), dim3(D256x256::THREADS),
                       0, s, (const uint8_t*)g.W, (const uint8_t*)g.X, g.scale_x, g.scale_w, g.Y, N, M, g.K, tiles_a,
                       tiles_b, (int)n_big, parts);
    return hipGetLastError();
}

template <class TL>
int64_t tiles_of(const DenseArgs& g) {
    return ((g.N + TL::BA - 1) / TL::BA) * ((g.M + TL::BB - 1) / TL::BB) * TL::OCC;
}

// The same tile choice as the sparse kernels: the largest tile that keeps
// most CUs busy (192 workgroups), else the smallest; a short last round of
// 256 x 256 tiles as quarter tiles (at most a quarter of the chip) or half
// tiles (at most half of it).
template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch(const DenseArgs& g, hipStream_t s, const char** kname) {
    constexpr int64_t kFill = 192;
    constexpr int64_t kCUs = 256;   // compute units of the gfx950 parts (MI350X, MI355X)
    if (g.M > 64) {
        const int64_t t256 = tiles_of<D256x256>(g), rest = t256 % kCUs;
        if (t256 > kCUs && rest > 0 && 4 * rest <= kCUs)
            return launch_tail<DT, OUT>(g, s, kname, t256 - rest, rest, 4);
        if (t256 > kCUs && rest > 0 && 2 * rest <= kCUs)
            return launch_tail<DT, OUT>(g, s, kname, t256 - rest, rest, 2);
        // between 256 x 256 and 256 x 128: the cheaper rounds, as the sparse kernels choose
        const int64_t t128 = tiles_of<D256x128>(g);
        const int64_t r256 = (t256 + kCUs - 1) / kCUs, r128 = (t128 + kCUs - 1) / kCUs;
        if (t256 >= kFill || (t128 >= kFill && 10 * r256 <= 7 * r128))
            return launch_tile<DT, OUT, D256x256>(g, s, kname, "dense_big_256x256");
        if (t128 >= kFill) return launch_tile<DT, OUT, D256x128>(g, s, kname, "dense_big_256x128");
        if (tiles_of<D128x128>(g) / D128x128::OCC >= kFill)
            return launch_tile<DT, OUT, D128x128>(g, s, kname, "dense_big_128x128");
        return launch_tile<DT, OUT, D128x64>(g, s, kname, "dense_big_128x64");
    }
    if (tiles_of<D256x64>(g) >= kFill) return launch_tile<DT, OUT, D256x64>(g, s, kname, "dense_big_256x64");
    return launch_tile<DT, OUT, D128x64>(g, s, kname, "dense_big_128x64");
}

}  // namespace

hipError_t launch_dense_gemm_big(const DenseArgs& g, hipStream_t s, const char** kname) {
    switch (g.in_dt) {
    case SP24_BF16:
        if (g.out_dt == SP24_BF16) return launch<SP24_BF16, SP24_BF16>(g, s, kname);
        if (g.out_dt == SP24_F16) return launch<SP24_BF16, SP24_F16>(g, s, kname);
        return launch<SP24_BF16, SP24_F32>(g, s, kname);
    case SP24_F16:
        if (g.out_dt == SP24_F16) return launch<SP24_F16, SP24_F16>(g, s, kname);
        if (g.out_dt == SP24_BF16) return launch<SP24_F16, SP24_BF16>(g, s, kname);
        return launch<SP24_F16, SP24_F32>(g, s, kname);
    case SP24_E4M3:
        if (g.out_dt == SP24_BF16) return launch<SP24_E4M3, SP24_BF16>(g, s, kname);
        return launch<SP24_E4M3, SP24_F32>(g, s, kname);
    case SP24_I8:
        if (g.out_dt == SP24_BF16) return launch<SP24_I8, SP24_BF16>(g, s, kname);
        return launch<SP24_I8, SP24_F32>(g, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
