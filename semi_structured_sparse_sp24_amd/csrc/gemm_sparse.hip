// gemm_sparse.hip -- 2:4 sparse x dense GEMM on gfx950 SMFMAC.
//
// Computes D[a][b] = sum_k A[a][k] * B[b][k], where A (RA x K) is the
// compressed operand (values + metadata) and B (RB x K) is dense; the result
// goes to Y[a * sya + b * syb].  With the weight compressed (A = W, B = X):
// sya = 1, syb = N, i.e. the kernel computes the tile of Y^T and stores it
// transposed; with the activation compressed (A = X, B = W): sya = N, syb = 1.
// Source of the operation: the 2:4-versus-quantization paper, section 2
// ("Sparse tensor cores": only the first operand is sparse, along the
// reduction axis; the indices select the matching elements of B).
//
// Two kernels:
//   skinny  few B rows (decode: M <= 64).  HBM-bound on the compressed
//           weight.  One workgroup owns 16 rows of A and all of B; its waves
//           split K (step s goes to wave s % waves), load operands straight
//           from global memory into registers (16-byte loads, each row's
//           bytes read once), and reduce their partial tiles through LDS in
//           a fixed order (deterministic, no atomics).
//   tiled   large M (prefill, dynamic operands).  Workgroup tile BA x BB,
//           K staged through double-buffered LDS one instruction step at a
//           time, 2 x 2 waves each owning (FA x FB) 16x16 fragments.
#include "mfma_ops.h"

namespace sp24 {
namespace {

// ------------------------------------------------------------------ skinny
constexpr int kMaxWaves = 16;

template <sp24_dtype DT, sp24_dtype OUT, int MT, int U>
__global__ void __launch_bounds__(kMaxWaves * 64)
sp24_skinny(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am,
            const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
            void* __restrict__ Y, int RA, int RB, int64_t K, int64_t sya, int64_t syb) {
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    __shared__ float red[kMaxWaves][MT][4][64];

    const int WAVES = blockDim.x >> 6;   // 4, 8 or 16: the waves split K
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int a0 = blockIdx.x * 16;
    const int steps = (int)(K / L::KSTEP);
    const uint32_t a_row_bytes = (uint32_t)(K / 2 * L::ELEM), b_row_bytes = (uint32_t)(K * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);

    // buffers sized to the operands: rows past RA / RB read as zeros
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);
    const Buf bufM(am, (uint32_t)RA * m_row_bytes);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);
    const uint32_t a_base = (uint32_t)(a0 + r) * a_row_bytes + L::a_off(kg);
    const uint32_t m_base = (uint32_t)(a0 + r) * m_row_bytes + 4 * L::meta_word(kg);
    const int msh = L::meta_shift(kg);
    uint32_t b_base[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        b_base[mt] = (uint32_t)(mt * 16 + r) * b_row_bytes;

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Each wave takes a contiguous chunk of K steps, so each of its rows is
    // read as one contiguous run; the whole K loop of a workgroup starts at a
    // rotated step so that concurrent workgroups read different column
    // offsets (rows are power-of-two strides apart).
    const int chunk = (steps + WAVES - 1) / WAVES;
    const int rot = (int)((blockIdx.x * 13u) % (unsigned)max(steps, 1));
    for (int i0 = 0; i0 < chunk; i0 += U) {
        uint4 a[U], b0[U][MT], b1[U][MT];
        uint32_t idx[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int sl = wave * chunk + i0 + u;
            live[u] = i0 + u < chunk && sl < steps;
            int s = sl + rot;
            s = s >= steps ? s - steps : s;
            const uint32_t sa_off = live[u] ? a_base + (uint32_t)s * L::A_STEP_BYTES : kOOB;
            const uint32_t sm_off = live[u] ? m_base + (uint32_t)s * (4 * L::META_WORDS) : kOOB;
            a[u] = bufA.ld16(sa_off);
            idx[u] = bufM.ld4(sm_off) >> msh;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const uint32_t o = live[u] ? b_base[mt] + (uint32_t)s * L::B_STEP_BYTES : kOOB;
                b0[u][mt] = bufB.ld16(o + L::b_off0(kg));
                b1[u][mt] = bufB.ld16(o + L::b_off1(kg));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (live[u]) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt] = Op::mma(a[u], b0[u][mt], b1[u][mt], idx[u], acc[mt]);
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[wave][mt][i][lane] = acc[mt][i];
    __syncthreads();

    // D[4*kg + i][l % 16] of fragment mt lives at red[.][mt][i][kg*16 + l%16]
    for (int o = threadIdx.x; o < 16 * 16 * MT; o += WAVES * 64) {
        const int al = o & 15, bl = o >> 4;
        const int mt = bl >> 4, ln = ((al >> 2) << 4) | (bl & 15), i = al & 3;
        float v = 0.f;
        for (int w = 0; w < WAVES; ++w)   // fixed order: deterministic
            v += red[w][mt][i][ln];
        const int ar = a0 + al, br = bl;
        if (ar < RA && br < RB) {
            if (sa)
                v *= sa[ar];
            if (sb)
                v *= sb[br];
            store_out<OUT>(Y, (int64_t)ar * sya + (int64_t)br * syb, v);
        }
    }
}

// ------------------------------------------------------------------ tiled
template <int FA, int FB>
struct TiledShape {
    static constexpr int BA = 2 * FA * 16;   // 2 waves along A
    static constexpr int BB = 2 * FB * 16;   // 2 waves along B
    static constexpr int A_STRIDE = 64 + 16; // bytes per A row in LDS (one step) + pad
    static constexpr int B_STRIDE = 128 + 16;
};

template <sp24_dtype DT, sp24_dtype OUT, int FA, int FB>
__global__ void __launch_bounds__(256)
sp24_tiled(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am,
           const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
           void* __restrict__ Y, int RA, int RB, int64_t K, int64_t sya, int64_t syb, int tiles_a) {
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    using S = TiledShape<FA, FB>;
    constexpr int BA = S::BA, BB = S::BB, MWS = L::META_WORDS;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BA * S::A_STRIDE];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BB * S::B_STRIDE];
    __shared__ uint32_t lds_m[2][BA * MWS];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, kg = lane >> 4;
    const int wa = wave >> 1, wb = wave & 1;
    const int ta = blockIdx.x % tiles_a, tb = blockIdx.x / tiles_a;
    const int a0 = ta * BA, b0 = tb * BB;
    const int steps = (int)(K / L::KSTEP);

    // global -> LDS assignment: A chunks of 16 B (4 per row), B chunks (8 per
    // row), metadata words.  Buffers are sized to the operands, so rows past
    // RA / RB read as zeros.
    const uint32_t a_row_bytes = (uint32_t)(K / 2 * L::ELEM), b_row_bytes = (uint32_t)(K * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);
    const Buf bufM(am, (uint32_t)RA * m_row_bytes);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);
    constexpr int A_CHUNKS = BA * 4 / 256, B_CHUNKS = BB * 8 / 256, M_WORDS = (BA * MWS + 255) / 256;
    uint32_t ga[A_CHUNKS];
    int la[A_CHUNKS];
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
        int c = tid + j * 256, row = c >> 2, col = c & 3;
        ga[j] = (uint32_t)(a0 + row) * a_row_bytes + col * 16;
        la[j] = row * S::A_STRIDE + col * 16;
    }
    uint32_t gb[B_CHUNKS];
    int lb[B_CHUNKS];
#pragma unroll
    for (int j = 0; j < B_CHUNKS; ++j) {
        int c = tid + j * 256, row = c >> 3, col = c & 7;
        gb[j] = (uint32_t)(b0 + row) * b_row_bytes + col * 16;
        lb[j] = row * S::B_STRIDE + col * 16;
    }
    uint32_t gm[M_WORDS];
    bool usem[M_WORDS];
#pragma unroll
    for (int j = 0; j < M_WORDS; ++j) {
        int c = tid + j * 256, row = c / MWS, w = c % MWS;
        usem[j] = c < BA * MWS;
        gm[j] = (uint32_t)(a0 + row) * m_row_bytes + 4 * w;
    }

    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    uint32_t rm[M_WORDS];
    // K loop starts at a per-workgroup rotated step (spreads concurrent
    // workgroups over memory channels; the sum order is fixed per shape)
    const int rot = (int)((blockIdx.x * 13u) % (unsigned)steps);
    auto gload = [&](int sl) {
        const uint32_t s = (uint32_t)(sl + rot >= steps ? sl + rot - steps : sl + rot);
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j)
            ra[j] = bufA.ld16(ga[j] + s * L::A_STEP_BYTES);
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j)
            rb[j] = bufB.ld16(gb[j] + s * L::B_STEP_BYTES);
#pragma unroll
        for (int j = 0; j < M_WORDS; ++j)
            rm[j] = bufM.ld4(usem[j] ? gm[j] + s * (4 * MWS) : kOOB);
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < A_CHUNKS; ++j)
            *reinterpret_cast<uint4*>(&lds_a[buf][la[j]]) = ra[j];
#pragma unroll
        for (int j = 0; j < B_CHUNKS; ++j)
            *reinterpret_cast<uint4*>(&lds_b[buf][lb[j]]) = rb[j];
#pragma unroll
        for (int j = 0; j < M_WORDS; ++j)
            if (usem[j])
                lds_m[buf][tid + j * 256] = rm[j];
    };

    f32x4 acc[FA][FB];
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
        for (int j = 0; j < FB; ++j)
            acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    gload(0);
    lstore(0);
    __syncthreads();
    const int msh = L::meta_shift(kg), mwd = L::meta_word(kg);
    for (int s = 0; s < steps; ++s) {
        const int buf = s & 1;
        if (s + 1 < steps)
            gload(s + 1);
        uint4 fa[FA];
        uint32_t fi[FA];
#pragma unroll
        for (int i = 0; i < FA; ++i) {
            int row = wa * FA * 16 + i * 16 + r;
            fa[i] = *reinterpret_cast<const uint4*>(&lds_a[buf][row * S::A_STRIDE + L::a_off(kg)]);
            fi[i] = lds_m[buf][row * MWS + mwd] >> msh;
        }
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            int row = wb * FB * 16 + j * 16 + r;
            uint4 fb0 = *reinterpret_cast<const uint4*>(&lds_b[buf][row * S::B_STRIDE + L::b_off0(kg)]);
            uint4 fb1 = *reinterpret_cast<const uint4*>(&lds_b[buf][row * S::B_STRIDE + L::b_off1(kg)]);
#pragma unroll
            for (int i = 0; i < FA; ++i)
                acc[i][j] = Op::mma(fa[i], fb0, fb1, fi[i], acc[i][j]);
        }
        if (s + 1 < steps)
            lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: fragment (i, j), lane -> D[a][b] with a = .. + 4*kg + q, b = .. + r
#pragma unroll
    for (int i = 0; i < FA; ++i) {
#pragma unroll
        for (int j = 0; j < FB; ++j) {
            const int ar = a0 + wa * FA * 16 + i * 16 + 4 * kg;
            const int br = b0 + wb * FB * 16 + j * 16 + r;
            if (br >= RB)
                continue;
            f32x4 v = acc[i][j];
            const float fsb = sb ? sb[br] : 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] *= (sa && ar + q < RA ? sa[ar + q] : 1.f) * fsb;
            const int64_t off = (int64_t)ar * sya + (int64_t)br * syb;
            if (sya == 1 && ar + 3 < RA && (off & 3) == 0) {
                store_out4<OUT>(Y, off, v);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (ar + q < RA)
                        store_out<OUT>(Y, off + (int64_t)q * sya, v[q]);
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch
template <sp24_dtype DT, sp24_dtype OUT>
hipError_t dispatch(const GemmArgs& g, hipStream_t s, const char** kname) {
    const int RA = (int)(g.a_is_w ? g.N : g.M);
    const int RB = (int)(g.a_is_w ? g.M : g.N);
    const int64_t sya = g.a_is_w ? 1 : g.N, syb = g.a_is_w ? g.N : 1;
    const uint8_t* av = (const uint8_t*)g.a_vals;
    const uint8_t* b = (const uint8_t*)g.b;
    const int tiles16 = (RA + 15) / 16;
    if (RB <= 64) {
        const int steps = (int)(g.K / SparseOp<DT>::KSTEP);
        // enough waves to cover the chip (>= ~8 per CU) without starving each wave of steps
        int waves = 16;
        while (waves > 4 && ((int64_t)tiles16 * waves > 8192 || steps < waves * 2))
            waves >>= 1;
#define SP24_SKINNY(MT, U)                                                                            \
    do {                                                                                              \
        hipLaunchKernelGGL((sp24_skinny<DT, OUT, MT, U>), dim3(tiles16), dim3(waves * 64), 0, s, av,    \
                           g.a_meta, b, g.scale_a, g.scale_b, g.Y, RA, RB, g.K, sya, syb);            \
        if (kname) *kname = "sp24_skinny_m" #MT;                                                      \
    } while (0)
        const int mt = (RB + 15) / 16;
        if (mt <= 1) SP24_SKINNY(1, 4);
        else if (mt == 2) SP24_SKINNY(2, 2);
        else SP24_SKINNY(4, 2);
#undef SP24_SKINNY
    } else if ((int64_t)((RA + 255) / 256) * ((RB + 255) / 256) >= 192) {
        return launch_sp24_gemm_big(g, s, kname);
    } else {
        constexpr int FA = 4, FB = 4;
        using S = TiledShape<FA, FB>;
        const int tiles_a = (RA + S::BA - 1) / S::BA, tiles_b = (RB + S::BB - 1) / S::BB;
        hipLaunchKernelGGL((sp24_tiled<DT, OUT, FA, FB>), dim3(tiles_a * tiles_b), dim3(256), 0, s, av,
                           g.a_meta, b, g.scale_a, g.scale_b, g.Y, RA, RB, g.K, sya, syb, tiles_a);
        if (kname) *kname = "sp24_tiled_128x128";
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sp24_gemm(const GemmArgs& g, hipStream_t s, const char** kname) {
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
