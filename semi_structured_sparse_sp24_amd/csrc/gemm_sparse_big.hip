// gemm_sparse_big.hip -- 2:4 sparse x dense GEMM for large M (prefill,
// dynamic operands) on gfx950 SMFMAC.
//
// Same contract as the kernels in gemm_sparse.hip: D[a][b] = sum_k A[a][k] *
// B[b][k] with A compressed (values + metadata) and B dense, stored to
// Y[a * sya + b * syb] (the paper's section 2, "Sparse tensor cores").
//
// Design (one workgroup per CU):
//   - tile 256 (A rows) x 256 (B rows); 8 waves in a 4 x 2 grid (two per
//     SIMD), each owning 64 x 128 = 4 x 8 fragments of v_smfmac_f32_16x16x64
//     (16-bit) or v_smfmac_f32_16x16x128 (fp8), accumulated in 128 registers
//     per lane.  (One wave per SIMD with 128 x 128 each needs 256 accumulator
//     registers plus operands, and the compiler then shuffles accumulators
//     between register files inside the loop; two waves per SIMD also hide
//     each other's LDS latency.)
//   - K advances one instruction step per stage: A 256 rows x 64 B, metadata
//     256 rows x 8 (or 16) B, B 256 rows x 128 B = 50 KB; three stages live
//     in LDS (150 KB of the 160 KB);
//   - the stages are filled by direct global->LDS loads (buffer_load_dwordx4
//     ... lds): no registers, no LDS write instructions; two steps are in
//     flight while the third is consumed, with one barrier per step;
//   - each wave-wide load writes 1 KiB of LDS in lane order, so the LDS
//     layout is chosen through which global chunk each lane fetches: the
//     16-byte chunks of a row are XOR-swizzled by row so that the fragment
//     reads (16 rows x 16 B per lane group) hit 16 distinct bank groups;
//   - workgroups are ordered so that the ones resident on one XCD at a time
//     form a 4 (A tiles) x 8 (B tiles) block that shares operands through
//     that XCD's L2.
#include "mfma_ops.h"

namespace sp24 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBA = 256, kBB = 256;
constexpr int kWA = 4, kWB = 2, kWaves = kWA * kWB, kThreads = 64 * kWaves;
constexpr int kFA = kBA / 16 / kWA, kFB = kBB / 16 / kWB;   // 16x16 fragments per wave: 4 x 8
constexpr int kAStage = kBA * 64;     // bytes of compressed A per stage
constexpr int kBStage = kBB * 128;    // bytes of dense B per stage

__device__ __forceinline__ void dma16(const Buf& b, void* lds_base, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (lds_void*)lds_base, 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ void dma4(const Buf& b, void* lds_base, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (lds_void*)lds_base, 4, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same, and every LDS read issued so far complete (lgkmcnt(0))
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

template <sp24_dtype DT, sp24_dtype OUT>
__global__ void __launch_bounds__(kThreads, 1)
sp24_big(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ B,
         const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ Y, int RA, int RB,
         int64_t K, int64_t sya, int64_t syb, int tiles_a, int tiles_b) {
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    constexpr int MWS = L::META_WORDS;                  // metadata words per row per step: 2 or 4
    constexpr int kMStage = kBA * MWS * 4;
    constexpr int A_LOADS = kAStage / 1024 / kWaves;    // per wave: 2
    constexpr int B_LOADS = kBStage / 1024 / kWaves;    // per wave: 4
    constexpr int M_LOADS = kMStage / 256 / kWaves;     // per wave (dword loads): 1 or 2
    constexpr int LOADS = A_LOADS + B_LOADS + M_LOADS;  // per wave per stage

    __shared__ __attribute__((aligned(1024))) uint8_t a0s[kAStage], a1s[kAStage], a2s[kAStage];
    __shared__ __attribute__((aligned(1024))) uint8_t b0s[kBStage], b1s[kBStage], b2s[kBStage];
    __shared__ __attribute__((aligned(1024))) uint8_t m0s[kMStage], m1s[kMStage], m2s[kMStage];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int r = lane & 15, kg = lane >> 4;
    const int wa = wave / kWB, wb = wave % kWB;

    // ---- tile order: XCD-aware, grouped 4 A tiles x all B tiles
    const int nwg = gridDim.x;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int per_xcd = (nwg + 7) >> 3, full = nwg & 7 ? (nwg & 7) : 8;   // XCDs holding per_xcd tiles
    const int t = xcd < full ? xcd * per_xcd + local : full * per_xcd + (xcd - full) * (per_xcd - 1) + local;
    constexpr int G = 4;
    const int group = t / (G * tiles_b), within = t - group * G * tiles_b;
    const int g_rows = min(G, tiles_a - group * G);
    const int ta = group * G + within % g_rows, tb = within / g_rows;
    const int a0 = ta * kBA, b0 = tb * kBB;

    const int steps = (int)(K / L::KSTEP);
    const uint32_t a_row_bytes = (uint32_t)(K / 2 * L::ELEM), b_row_bytes = (uint32_t)(K * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);     // rows past RA / RB read as zeros
    const Buf bufM(am, (uint32_t)RA * m_row_bytes);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);

    // ---- per-lane global offsets of this wave's loads (step 0), and LDS slots
    uint32_t ga[A_LOADS], gb[B_LOADS], gm[M_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = 16 * (A_LOADS * wave + j) + (lane >> 2);
        const int c = (lane & 3) ^ ((row >> 1) & 3);             // chunk stored in slot lane & 3
        ga[j] = (uint32_t)(a0 + row) * a_row_bytes + 16 * c;
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int row = 8 * (B_LOADS * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        gb[j] = (uint32_t)(b0 + row) * b_row_bytes + 16 * c;
    }
#pragma unroll
    for (int j = 0; j < M_LOADS; ++j) {
        const int w = 64 * (M_LOADS * wave + j) + lane;           // metadata word of the stage
        gm[j] = (uint32_t)(a0 + w / MWS) * m_row_bytes + 4 * (w % MWS);
    }

    // K loop start rotated per group of tile-sharing workgroups: members of a
    // group (resident together on one XCD) walk K in step and share operand
    // slices through L2, while different groups spread over memory channels
    const int rot = (int)(((unsigned)group * 13u) % (unsigned)steps);
    auto issue = [&](uint8_t* as, uint8_t* bs, uint8_t* ms, int sl) {
        // step sl of the rotated K loop; steps past the end load nothing useful
        int s = sl + rot;
        s = s >= steps ? s - steps : s;
        const bool live = sl < steps;
        const uint32_t sA = live ? (uint32_t)s * L::A_STEP_BYTES : kOOB;
        const uint32_t sB = live ? (uint32_t)s * L::B_STEP_BYTES : kOOB;
        const uint32_t sM = live ? (uint32_t)s * (4 * MWS) : kOOB;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j)
            dma16(bufA, as + 1024 * (A_LOADS * wave + j), ga[j], sA);
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j)
            dma16(bufB, bs + 1024 * (B_LOADS * wave + j), gb[j], sB);
#pragma unroll
        for (int j = 0; j < M_LOADS; ++j)
            dma4(bufM, ms + 256 * (M_LOADS * wave + j), gm[j], sM);
    };

    // ---- fragment read offsets (bytes within a stage)
    const int a_frag = (wa * 16 * kFA + r) * 64 + 16 * (kg ^ ((r >> 1) & 3));
    const int m_frag = ((wa * 16 * kFA + r) * MWS + L::meta_word(kg)) * 4;
    const int msh = L::meta_shift(kg);
    const int b_frag0 = (wb * 16 * kFB + r) * 128 + 16 * (kg ^ ((r >> 1) & 7));
    const int b_frag1 = (wb * 16 * kFB + r) * 128 + 16 * ((4 + kg) ^ ((r >> 1) & 7));

    f32x4 acc[kFA][kFB];
#pragma unroll
    for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int j = 0; j < kFB; ++j)
            acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t* as, const uint8_t* bs, const uint8_t* ms) {
        uint4 fa[kFA];
        uint32_t fi[kFA];
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
            fa[i] = *reinterpret_cast<const uint4*>(as + a_frag + i * 16 * 64);
            fi[i] = *reinterpret_cast<const uint32_t*>(ms + m_frag + i * 16 * MWS * 4) >> msh;
        }
#pragma unroll
        for (int j = 0; j < kFB; ++j) {
            const uint4 fb0 = *reinterpret_cast<const uint4*>(bs + b_frag0 + j * 16 * 128);
            const uint4 fb1 = *reinterpret_cast<const uint4*>(bs + b_frag1 + j * 16 * 128);
#pragma unroll
            for (int i = 0; i < kFA; ++i)
                acc[i][j] = Op::mma(fa[i], fb0, fb1, fi[i], acc[i][j]);
        }
    };

    // ---- pipeline: stages 0 and 1 in flight, then one step per stage
    // block.  Before each block a wave waits for its own loads of the stage
    // it is about to read (the next stage's may stay in flight) and for its
    // LDS reads of the previous stage, then a barrier makes every wave's
    // loads visible and frees the stage the new loads overwrite.  The step
    // count is padded to a multiple of 3 (padded steps read zeros) so the loop
    // body has no exits: that keeps the accumulators in registers.
    issue(a0s, b0s, m0s, 0);
    issue(a1s, b1s, m1s, 1);
    const int steps3 = (steps + 2) / 3 * 3;
    for (int s = 0; s < steps3; s += 3) {
        wait_vmcnt_lgkm0<LOADS>();
        __builtin_amdgcn_s_barrier();
        issue(a2s, b2s, m2s, s + 2);
        compute(a0s, b0s, m0s);
        wait_vmcnt_lgkm0<LOADS>();
        __builtin_amdgcn_s_barrier();
        issue(a0s, b0s, m0s, s + 3);
        compute(a1s, b1s, m1s);
        wait_vmcnt_lgkm0<LOADS>();
        __builtin_amdgcn_s_barrier();
        issue(a1s, b1s, m1s, s + 4);
        compute(a2s, b2s, m2s);
    }
    wait_vmcnt<0>();   // drain the (useless) loads of steps past the end

    // ---- epilogue: fragment (i, j), lane -> D[a][b], a = .. + 4*kg + q, b = .. + r
#pragma unroll
    for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int j = 0; j < kFB; ++j) {
            const int ar = a0 + wa * 16 * kFA + i * 16 + 4 * kg;
            const int br = b0 + wb * 16 * kFB + j * 16 + r;
            if (br >= RB || ar >= RA)
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

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_big(const GemmArgs& g, hipStream_t s, const char** kname) {
    const int RA = (int)(g.a_is_w ? g.N : g.M);
    const int RB = (int)(g.a_is_w ? g.M : g.N);
    const int64_t sya = g.a_is_w ? 1 : g.N, syb = g.a_is_w ? g.N : 1;
    const int tiles_a = (RA + kBA - 1) / kBA, tiles_b = (RB + kBB - 1) / kBB;
    if (kname)
        *kname = "sp24_big_256x256";
    if (g.dry)
        return hipSuccess;
    hipLaunchKernelGGL((sp24_big<DT, OUT>), dim3(tiles_a * tiles_b), dim3(kThreads), 0, s,
                       (const uint8_t*)g.a_vals, g.a_meta, (const uint8_t*)g.b, g.scale_a, g.scale_b, g.Y, RA,
                       RB, g.K, sya, syb, tiles_a, tiles_b);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sp24_gemm_big(const GemmArgs& g, hipStream_t s, const char** kname) {
    switch (g.in_dt) {
    case SP24_BF16:
        if (g.out_dt == SP24_BF16) return launch_big<SP24_BF16, SP24_BF16>(g, s, kname);
        if (g.out_dt == SP24_F16) return launch_big<SP24_BF16, SP24_F16>(g, s, kname);
        return launch_big<SP24_BF16, SP24_F32>(g, s, kname);
    case SP24_F16:
        if (g.out_dt == SP24_F16) return launch_big<SP24_F16, SP24_F16>(g, s, kname);
        if (g.out_dt == SP24_BF16) return launch_big<SP24_F16, SP24_BF16>(g, s, kname);
        return launch_big<SP24_F16, SP24_F32>(g, s, kname);
    case SP24_E4M3:
        if (g.out_dt == SP24_BF16) return launch_big<SP24_E4M3, SP24_BF16>(g, s, kname);
        return launch_big<SP24_E4M3, SP24_F32>(g, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
