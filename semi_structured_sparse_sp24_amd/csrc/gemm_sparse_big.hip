// gemm_sparse_big.hip -- 2:4 sparse x dense GEMM for large outputs (prefill,
// dynamic operands, and the 17-64 row decode cases) on gfx950 SMFMAC.
//
// Same contract as the kernels in gemm_sparse.hip: D[a][b] = sum_k A[a][k] *
// B[b][k] with A compressed (values + metadata) and B dense, stored to
// Y[a * sya + b * syb] (the paper's section 2, "Sparse tensor cores").
//
// Design (shown for the 256 x 256 tile; smaller tiles for outputs that would
// not fill the chip follow the same plan with fewer rows):
//   - tile 256 (A rows) x 256 (B rows); 8 waves in a 2 x 4 grid (two per
//     SIMD), each owning 128 x 64 = 8 x 4 fragments of v_smfmac_f32_16x16x64
//     (16-bit) or v_smfmac_f32_16x16x128 (fp8), accumulated in 128 registers
//     per lane.  Every wave reads its A and B rows from LDS each step, so the
//     grid sets the LDS read traffic: 2 x 4 reads the half-width A four
//     times and B twice, 128 KiB per step, where 4 x 2 reads 160 KiB (and
//     runs 4% slower).  (One wave per SIMD with 128 x 128 each needs 256
//     accumulator registers plus operands, and the compiler then shuffles
//     accumulators between register files inside the loop; two waves per
//     SIMD also hide each other's LDS latency.)
//   - K advances one instruction step per stage: A 256 rows x 64 B and B 256
//     rows x 128 B; metadata comes in blocks of 32 B per row (four 16-bit
//     steps, or two fp8 steps); three stages and two metadata blocks fill
//     the 160 KB of LDS;
//   - the stages are filled by direct global->LDS loads (buffer_load_dwordx4
//     ... lds): no registers, no LDS write instructions; two steps are in
//     flight while the third is consumed, with one barrier per step;
//   - each wave-wide load writes 1 KiB of LDS in lane order, so the LDS
//     layout is chosen through which global chunk each lane fetches: the
//     16-byte chunks of a row are XOR-swizzled by row so that the fragment
//     reads (16 rows x 16 B per lane group) hit 16 distinct bank groups;
//   - workgroups are ordered so that the ones resident on one XCD at a time
//     (32) form an 8 (A tiles) x 4 (B tiles) block that shares operands
//     through that XCD's L2;
//   - a grid whose last round would leave most of the chip idle runs that
//     round as quarter tiles (sp24_big_tail).
#include "mfma_ops.h"

namespace sp24 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// Metadata in LDS: blocks of kMetaRow bytes per A row (four 16-bit steps, or
// two fp8 steps), in a ring of kMetaSlots blocks.
constexpr int kMetaRow = 32, kMetaSlots = 2;

// Tile shapes: BA rows of A x BB rows of B, WA x WB waves, OCC workgroups per CU.
template <int BA_, int BB_, int WA_, int WB_, int OCC_>
struct Tile {
    static constexpr int BA = BA_, BB = BB_, WA = WA_, WB = WB_, OCC = OCC_;
    static constexpr int WAVES = WA * WB, THREADS = 64 * WAVES;
    static constexpr int FA = BA / 16 / WA, FB = BB / 16 / WB;   // 16x16 fragments per wave
    static constexpr int A_STAGE = BA * 64;    // bytes of compressed A per stage
    static constexpr int B_STAGE = BB * 128;   // bytes of dense B per stage
    static constexpr int M_BLOCK = BA * kMetaRow;   // bytes of one metadata block
};
using T256x256 = Tile<256, 256, 2, 4, 1>;
using T256x128 = Tile<256, 128, 4, 2, 1>;
using T128x128 = Tile<128, 128, 2, 4, 2>;
using T256x64 = Tile<256, 64, 4, 2, 1>;
using T128x64 = Tile<128, 64, 4, 2, 2>;

__device__ __forceinline__ void dma16(const Buf& b, void* lds_base, uint32_t voff, uint32_t soff) {
    dma16_lds(b, lds_base, voff, soff);
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

// The two 2:4 halves of dense A rows, for the dense tiles of the hybrid GEMM:
// any group of four is the sum of two groups of two, [a b 0 0] + [0 0 c d],
// and each is a 2:4 group with fixed positions (0, 1) and (2, 3).  q0, q1 are
// a lane's 32 dense bytes of one step (its SMFMAC lane range of dense K);
// lo gets the values at positions 0, 1 of every group, hi those at 2, 3.
template <sp24_dtype DT>
__device__ __forceinline__ void split_halves(const uint4& q0, const uint4& q1, uint4& lo, uint4& hi) {
    if constexpr (SparseOp<DT>::ELEM == 1) {
        // a group is one dword: bytes 0, 1 and bytes 2, 3
        lo = make_uint4(__builtin_amdgcn_perm(q0.y, q0.x, 0x05040100u), __builtin_amdgcn_perm(q0.w, q0.z, 0x05040100u),
                        __builtin_amdgcn_perm(q1.y, q1.x, 0x05040100u), __builtin_amdgcn_perm(q1.w, q1.z, 0x05040100u));
        hi = make_uint4(__builtin_amdgcn_perm(q0.y, q0.x, 0x07060302u), __builtin_amdgcn_perm(q0.w, q0.z, 0x07060302u),
                        __builtin_amdgcn_perm(q1.y, q1.x, 0x07060302u), __builtin_amdgcn_perm(q1.w, q1.z, 0x07060302u));
    } else {
        // a group is two dwords: the first holds positions 0, 1, the second 2, 3
        lo = make_uint4(q0.x, q0.z, q1.x, q1.z);
        hi = make_uint4(q0.y, q0.w, q1.y, q1.w);
    }
}

// The dense K range of a K-split weight: one 16x16 dense MFMA per fragment
// and half step, a half step being 64 bytes of a row (32 16-bit or 64 8-bit
// elements).  A lane supplies the 16 bytes at 16 * kg of its A row and of its
// B row; the instructions only need A and B to assign K to (lane group, byte)
// alike, which they do.  The output layout is that of the 16x16 SMFMAC, so
// both ranges accumulate into the same registers.  fp8 has no dense 16x16
// instruction taking 16 bytes a lane: two 8-byte ones (16x16x32) stand in.
template <sp24_dtype DT>
struct DenseHalf;
template <>
struct DenseHalf<SP24_BF16> {
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};
template <>
struct DenseHalf<SP24_F16> {
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};
template <>
struct DenseHalf<SP24_I8> {
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        i32x4 ci = __builtin_bit_cast(i32x4, c);
        ci = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), ci, 0,
                                                   0, 0);
        return __builtin_bit_cast(f32x4, ci);
    }
};
template <>
struct DenseHalf<SP24_E4M3> {
    __device__ static __forceinline__ f32x4 mma(uint4 a, uint4 b, f32x4 c) {
        const long a0 = (long)(((uint64_t)a.y << 32) | a.x), a1 = (long)(((uint64_t)a.w << 32) | a.z);
        const long b0 = (long)(((uint64_t)b.y << 32) | b.x), b1 = (long)(((uint64_t)b.w << 32) | b.z);
        c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, c, 0, 0, 0);
    }
};

// One output tile of the GEMM, D[a][b] for a in [a0, a0 + rows), b in
// [b0, b0 + TL::BB), over the whole K.  DENSE == false: A is compressed
// (values + metadata), tile rows TL::BA.  DENSE == true: A is dense and the
// tile has TL::BA / 2 rows, so that a step of dense A takes the bytes of a
// compressed step; each fragment runs two SMFMACs, one per 2:4 half, with
// constant positions.  The pipeline, the B side and the epilogue are the same.
// Y, sa and RA refer to this tile's region of A rows; `group` is the tile's
// group of tile-sharing workgroups (it sets the K rotation).
// KSPLIT: A's rows continue past the compressed range [0, K) with a dense
// range of KD more columns (ad: RA x KD, row-major), which B's rows (K + KD
// long) continue alike; after the compressed steps the tile runs the dense
// range in 64-byte half steps into the same accumulators.
template <sp24_dtype DT, sp24_dtype OUT, class TL, bool DENSE, bool KSPLIT = false>
__device__ __forceinline__ void tile_body(uint8_t* asb, uint8_t* bsb, uint8_t* msb,
                                          const uint8_t* __restrict__ av, const uint32_t* __restrict__ am,
                                          const uint8_t* __restrict__ B, const float* __restrict__ sa,
                                          const float* __restrict__ sb, void* __restrict__ Y, int RA, int RB,
                                          int64_t K, int64_t sya, int64_t syb, int a0, int b0, int group,
                                          const uint8_t* __restrict__ ad = nullptr, int64_t KD = 0) {
    static_assert(!(DENSE && KSPLIT), "a K-split tile has compressed rows");
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    constexpr int MWS = L::META_WORDS;                  // metadata words per row per step: 2 or 4
    // metadata goes in blocks of kMetaRow bytes per row: T steps (4 for
    // 16-bit, 2 for fp8).  Each row of a block is one request to L2, which
    // costs about as much as a full line of A or B: the fewer blocks, the
    // fewer requests (per-step 4-byte loads cost one per row and step).
    constexpr int T = kMetaRow / (4 * MWS);
    // a block slot is reloaded T * kMetaSlots steps after its previous load,
    // which must be at least 3 (the steps in flight) for its last reader to
    // have passed the barrier that precedes the reload
    static_assert(T * kMetaSlots >= 3, "metadata ring too short");
    constexpr int kBA = DENSE ? TL::BA / 2 : TL::BA;    // A rows of this tile
    constexpr int kBB = TL::BB, kWB = TL::WB, kWaves = TL::WAVES, kFB = TL::FB;
    constexpr int kFA = kBA / 16 / TL::WA;
    constexpr int kAStage = TL::A_STAGE, kBStage = TL::B_STAGE, kMBlock = TL::M_BLOCK;
    constexpr int M_WAVES = kMBlock / 1024;             // waves that issue a block's 1 KiB loads
    constexpr int A_LOADS = kAStage / 1024 / kWaves;    // per wave
    constexpr int B_LOADS = kBStage / 1024 / kWaves;    // per wave
    static_assert(A_LOADS * kWaves * 1024 == kAStage && B_LOADS * kWaves * 1024 == kBStage, "whole loads per wave");
    static_assert(M_WAVES * 1024 == kMBlock && M_WAVES <= kWaves, "metadata block");
    static_assert(kFA >= 1, "fragments per wave");
    // a dense A step is a B-sized row step: the stage then holds kBA rows of it
    constexpr int A_ROW_STEP = DENSE ? L::B_STEP_BYTES : L::A_STEP_BYTES;
    static_assert(kBA * A_ROW_STEP == kAStage, "dense rows fill the A stage");
    constexpr int A_CH = A_ROW_STEP / 16;               // 16-byte chunks per row step: 4, or 8 dense
    constexpr bool META = !DENSE;
    constexpr int AB = A_LOADS + B_LOADS;
    constexpr int U = T;                                // loop unroll: one metadata block

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int r = lane & 15, kg = lane >> 4;
    const int wa = wave / kWB, wb = wave % kWB;

    const int steps = (int)(K / L::KSTEP);
    const uint32_t a_row_bytes = (uint32_t)(DENSE ? K * L::ELEM : K / 2 * L::ELEM);
    const uint32_t b_row_bytes = (uint32_t)((K + (KSPLIT ? KD : 0)) * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);     // rows past RA / RB read as zeros
    const Buf bufM(am, META ? (uint32_t)RA * m_row_bytes : 0u);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);

    // ---- per-lane global offsets of this wave's loads (step 0), and LDS slots
    uint32_t ga[A_LOADS], gb[B_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        // a 1 KiB load covers 1024 / A_ROW_STEP rows; chunk c of a row lands in slot c ^ swizzle(row)
        const int row = (1024 / A_ROW_STEP) * (A_LOADS * wave + j) + lane / A_CH;
        const int c = (lane % A_CH) ^ ((row >> 1) & (A_CH - 1));
        ga[j] = (uint32_t)(a0 + row) * a_row_bytes + 16 * c;
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int row = 8 * (B_LOADS * wave + j) + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        gb[j] = (uint32_t)(b0 + row) * b_row_bytes + 16 * c;
    }
    // metadata: wave w < M_WAVES loads M_RPL rows of a block, M_CPR chunks of
    // 16 bytes each; in LDS the two chunks of a row trade places on every
    // other group of 8 rows, so that the 16 rows a fragment reads fall in 16
    // different 16-byte bank groups
    constexpr int M_CPR = kMetaRow / 16, M_RPL = 1024 / kMetaRow;
    static_assert(M_CPR == 1 || M_CPR == 2, "metadata chunks per row");
    auto m_swz = [](int row) { return M_CPR == 2 ? (row >> 3) & 1 : 0; };
    const int m_ld_row = M_RPL * min(wave, M_WAVES - 1) + lane / M_CPR;
    const uint32_t gm = (uint32_t)(a0 + m_ld_row) * m_row_bytes + 16 * ((lane % M_CPR) ^ m_swz(m_ld_row));

    // K loop start rotated per group of tile-sharing workgroups: members of a
    // group (resident together on one XCD) walk K in step and share operand
    // slices through L2, while different groups spread over memory channels.
    // The rotation keeps metadata blocks aligned (a multiple of T), and is
    // dropped when the step count is not a multiple of T.
    const int rot = (steps == 0 || steps % T) ? 0 : (int)(((unsigned)group * 13u) % (unsigned)(steps / T)) * T;
    auto issue_part = [&](uint8_t* as, uint8_t* bs, uint8_t* ms, int sl, bool do_a, bool do_bm) {
        // step sl of the rotated K loop; steps past the end load nothing useful
        int s = sl + rot;
        s = s >= steps ? s - steps : s;
        const bool live = sl < steps;
        const uint32_t sA = live ? (uint32_t)s * A_ROW_STEP : kOOB;
        const uint32_t sB = live ? (uint32_t)s * L::B_STEP_BYTES : kOOB;
        if (do_a) {
#pragma unroll
            for (int j = 0; j < A_LOADS; ++j)
                dma16(bufA, as + 1024 * (A_LOADS * wave + j), ga[j], sA);
        }
        if (do_bm) {
#pragma unroll
            for (int j = 0; j < B_LOADS; ++j)
                dma16(bufB, bs + 1024 * (B_LOADS * wave + j), gb[j], sB);
            // the block of steps s .. s + T - 1 (with a step count that T does
            // not divide, the last block's tail is past the row: read, never used)
            if (META && ms != nullptr && wave < M_WAVES)
                dma16(bufM, ms + 1024 * wave, gm, live ? (uint32_t)s * (4 * MWS) : kOOB);
        }
    };
    auto issue = [&](uint8_t* as, uint8_t* bs, uint8_t* ms, int sl) { issue_part(as, bs, ms, sl, true, true); };
    // before computing step x: this wave's loads of step x have landed when
    // only those of step x + 1 (issued one step later) may be outstanding
    auto wait_step = [&](bool next_has_meta) {
        if (META && next_has_meta && wave < M_WAVES)
            wait_vmcnt_lgkm0<AB + 1>();
        else
            wait_vmcnt_lgkm0<AB>();
    };

    // ---- fragment read offsets (bytes within a stage / a metadata block)
    const int a_row = wa * 16 * kFA + r;
    const int a_frag = a_row * 64 + 16 * (kg ^ ((r >> 1) & 3));
    // dense rows: the lane's 32 bytes are chunks 2 kg and 2 kg + 1 of its row
    const int a_frag_d0 = a_row * 128 + 16 * ((2 * kg) ^ ((r >> 1) & 7));
    const int a_frag_d1 = a_row * 128 + 16 * ((2 * kg + 1) ^ ((r >> 1) & 7));
    // the lane's metadata word in chunk 0 or 1 of its row (before the step's offset)
    const int m_frag0 = a_row * kMetaRow + 16 * (0 ^ m_swz(a_row)) + 4 * L::meta_word(kg);
    const int m_frag1 = a_row * kMetaRow + 16 * (1 ^ m_swz(a_row)) + 4 * L::meta_word(kg);
    const int msh = L::meta_shift(kg);
    const int b_frag0 = (wb * 16 * kFB + r) * 128 + 16 * (kg ^ ((r >> 1) & 7));
    const int b_frag1 = (wb * 16 * kFB + r) * 128 + 16 * ((4 + kg) ^ ((r >> 1) & 7));
    // positions (0, 1) and (2, 3) in every group: nibbles 0x4 and 0xE
    constexpr uint32_t kIdxLo = L::ELEM == 2 ? 0x4444u : 0x44444444u;
    constexpr uint32_t kIdxHi = L::ELEM == 2 ? 0xEEEEu : 0xEEEEEEEEu;

    f32x4 acc[kFA][kFB];
#pragma unroll
    for (int i = 0; i < kFA; ++i)
#pragma unroll
        for (int j = 0; j < kFB; ++j)
            acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // u: the step's position within its metadata block
    uint4 fa[kFA], fh[DENSE ? kFA : 1];
    uint32_t fi[kFA];
    auto load_a = [&](const uint8_t* as, const uint8_t* ms, int u) {
#pragma unroll
        for (int i = 0; i < kFA; ++i) {
            if constexpr (DENSE) {
                const uint4 q0 = *reinterpret_cast<const uint4*>(as + a_frag_d0 + i * 16 * 128);
                const uint4 q1 = *reinterpret_cast<const uint4*>(as + a_frag_d1 + i * 16 * 128);
                split_halves<DT>(q0, q1, fa[i], fh[i]);
            } else {
                fa[i] = *reinterpret_cast<const uint4*>(as + a_frag + i * 16 * 64);
                // step u's words start at word MWS u of the row's block
                const int mo = (((MWS * u) >> 2) ? m_frag1 : m_frag0) + 4 * ((MWS * u) & 3);
                fi[i] = *reinterpret_cast<const uint32_t*>(ms + mo + i * 16 * kMetaRow) >> msh;
            }
        }
    };
    // One step's MFMAs, the B fragments read one column ahead of their use
    // (two register slots), with the next stage's loads issued in two parts
    // along the way (A loads before the first MFMA, B and metadata halfway).
    auto compute_step = [&](const uint8_t* bs, auto&& issue_a, auto&& issue_bm) {
        uint4 b0[2], b1[2];
        b0[0] = *reinterpret_cast<const uint4*>(bs + b_frag0);
        b1[0] = *reinterpret_cast<const uint4*>(bs + b_frag1);
        issue_a();
#pragma unroll
        for (int j = 0; j < kFB; ++j) {
            if (j + 1 < kFB) {
                b0[(j + 1) & 1] = *reinterpret_cast<const uint4*>(bs + b_frag0 + (j + 1) * 16 * 128);
                b1[(j + 1) & 1] = *reinterpret_cast<const uint4*>(bs + b_frag1 + (j + 1) * 16 * 128);
            }
            if (j == kFB / 2)
                issue_bm();
#pragma unroll
            for (int i = 0; i < kFA; ++i) {
                if constexpr (DENSE) {
                    acc[i][j] = Op::mma(fa[i], b0[j & 1], b1[j & 1], kIdxLo, acc[i][j]);
                    acc[i][j] = Op::mma(fh[i], b0[j & 1], b1[j & 1], kIdxHi, acc[i][j]);
                } else {
                    acc[i][j] = Op::mma(fa[i], b0[j & 1], b1[j & 1], fi[i], acc[i][j]);
                }
            }
        }
    };

    // ---- pipeline: steps x and x + 1 in flight while x - 1 is consumed; one
    // barrier per step.  Before each step a wave waits for its own loads of
    // that step and for its LDS reads of the previous one; the barrier makes
    // every wave's loads visible and frees the stage the new loads overwrite.
    // Stage of step x: x % 3; metadata slot of step x: (x / T) % kMetaSlots,
    // loaded with the stage of its first step.  The stage and the slot are
    // run-time offsets; the loop runs T steps per iteration (padded steps
    // read zeros), so that where a block starts is static and the body has
    // no exits, which keeps the accumulators in registers.
    auto sa_ = [&](int st) { return asb + st * kAStage; };
    auto sb_ = [&](int st) { return bsb + st * kBStage; };
    auto ms_ = [&](int blk) { return msb + (blk % kMetaSlots) * kMBlock; };
    issue(sa_(0), sb_(0), ms_(0), 0);
    issue(sa_(1), sb_(1), 1 % T ? nullptr : ms_(1 / T), 1);
    const int stepsU = (steps + U - 1) / U * U;
    int st = 0;   // stage of step s
    for (int s = 0; s < stepsU; s += U) {
        const int blk = s / T;   // metadata block of steps s .. s + T - 1
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wait_step((u + 1) % T == 0);
            barrier_lds();
            const int x2 = u + 2;   // issued now: position within the unrolled block
            const int st2 = st == 0 ? 2 : st - 1;   // (s + u + 2) % 3
            uint8_t* const nms = x2 % T ? nullptr : ms_(blk + x2 / T);
            uint8_t* const nas = sa_(st2);
            uint8_t* const nbs = sb_(st2);
            load_a(sa_(st), ms_(blk + u / T), u % T);
            compute_step(sb_(st), [&] { issue_part(nas, nbs, nms, s + x2, true, false); },
                         [&] { issue_part(nas, nbs, nms, s + x2, false, true); });
            st = st == 2 ? 0 : st + 1;
        }
    }
    wait_vmcnt<0>();   // drain the (useless) loads of steps past the end

    if constexpr (KSPLIT) {
        // ---- the dense K range: half steps of HB bytes of every A and B row, through the same
        // three stages (A: BA rows x HB, the whole A stage; B: BB rows x HB, the first half of a B
        // stage), two half steps in flight, one barrier per half step; the 16-byte chunks of a row
        // XOR-swizzled by row as the compressed A rows are
        constexpr int HB = 64;
        constexpr int DA_BYTES = kBA * HB, DB_BYTES = kBB * HB;
        static_assert(DA_BYTES == kAStage && DB_BYTES <= kBStage, "a dense half step fits the stages");
        constexpr int DA_LOADS = DA_BYTES / 1024 / kWaves;
        constexpr int DB_WAVES = DB_BYTES / 1024 < kWaves ? DB_BYTES / 1024 : kWaves;
        constexpr int DB_LOADS = DB_BYTES / 1024 / DB_WAVES;
        static_assert(DA_LOADS >= 1 && DA_LOADS * kWaves * 1024 == DA_BYTES, "whole dense A loads per wave");
        static_assert(DB_LOADS * DB_WAVES * 1024 == DB_BYTES, "whole dense B loads");
        const int dsteps = (int)(KD * L::ELEM / HB);
        const uint32_t ad_row_bytes = (uint32_t)(KD * L::ELEM);
        const Buf bufD(ad, (uint32_t)RA * ad_row_bytes);   // rows past RA read as zeros
        uint32_t gd[DA_LOADS], gbd[DB_LOADS];
#pragma unroll
        for (int j = 0; j < DA_LOADS; ++j) {
            const int row = 16 * (DA_LOADS * wave + j) + lane / 4;
            gd[j] = (uint32_t)(a0 + row) * ad_row_bytes + 16 * ((lane & 3) ^ ((row >> 1) & 3));
        }
        const int wb_ld = min(wave, DB_WAVES - 1);
#pragma unroll
        for (int j = 0; j < DB_LOADS; ++j) {
            const int row = 16 * (DB_LOADS * wb_ld + j) + lane / 4;
            gbd[j] = (uint32_t)(b0 + row) * b_row_bytes + (uint32_t)(K * L::ELEM) + 16 * ((lane & 3) ^ ((row >> 1) & 3));
        }
        const int drot = dsteps > 0 ? (int)(((unsigned)group * 13u) % (unsigned)dsteps) : 0;
        auto dissue = [&](int st_, int hl) {
            int h = hl + drot;
            h = h >= dsteps ? h - dsteps : h;
            const uint32_t so = hl < dsteps ? (uint32_t)h * HB : kOOB;
#pragma unroll
            for (int j = 0; j < DA_LOADS; ++j)
                dma16(bufD, asb + st_ * kAStage + 1024 * (DA_LOADS * wave + j), gd[j], so);
            if (wave < DB_WAVES) {
#pragma unroll
                for (int j = 0; j < DB_LOADS; ++j)
                    dma16(bufB, bsb + st_ * kBStage + 1024 * (DB_LOADS * wave + j), gbd[j], so);
            }
        };
        const int a_fr = (wa * 16 * kFA + r) * HB + 16 * (kg ^ ((r >> 1) & 3));
        const int b_fr = (wb * 16 * kFB + r) * HB + 16 * (kg ^ ((r >> 1) & 3));
        // every wave is done reading the stages of the compressed range
        __syncthreads();
        if (dsteps > 0) {
            dissue(0, 0);
            dissue(1, 1);
        }
        int dst = 0;
        for (int hs = 0; hs < dsteps; ++hs) {
            if (wave < DB_WAVES)
                wait_vmcnt_lgkm0<DA_LOADS + DB_LOADS>();
            else
                wait_vmcnt_lgkm0<DA_LOADS>();
            barrier_lds();
            dissue(dst == 0 ? 2 : dst - 1, hs + 2);
            const uint8_t* as = asb + dst * kAStage;
            const uint8_t* bs = bsb + dst * kBStage;
            uint4 fb[kFB];
#pragma unroll
            for (int j = 0; j < kFB; ++j)
                fb[j] = *reinterpret_cast<const uint4*>(bs + b_fr + j * 16 * HB);
#pragma unroll
            for (int i = 0; i < kFA; ++i) {
                const uint4 fa_ = *reinterpret_cast<const uint4*>(as + a_fr + i * 16 * HB);
#pragma unroll
                for (int j = 0; j < kFB; ++j)
                    acc[i][j] = DenseHalf<DT>::mma(fa_, fb[j], acc[i][j]);
            }
            dst = dst == 2 ? 0 : dst + 1;
        }
        wait_vmcnt<0>();
    }

    // ---- epilogue: fragment (i, j), lane -> D[a][b], a = .. + 4*kg + q, b = .. + r
    auto value = [&](int i, int j, int ar, int br) {
        f32x4 v = acc_to_f32<DT>(acc[i][j]);
        const float fsb = sb ? sb[br] : 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[q] *= (sa && ar + q < RA ? sa[ar + q] : 1.f) * fsb;
        return v;
    };
    if constexpr (OUT != SP24_F32) {
        // A lane's fragment holds four consecutive rows of A in one column b.
        // When A indexes the output's contiguous dimension (sya == 1: the
        // transposed store of a weight-compressed GEMM) a store instruction
        // writes 8-byte pieces of 16 output rows; when B does (syb == 1: an
        // activation-compressed GEMM), 2-byte elements, one instruction per
        // row of A.  A whole block of the wave (EA rows of A x EB of B) is
        // instead staged in the stage memory the K loop no longer needs, one
        // output row after another, and written back as whole 16-byte pieces,
        // CPR lanes per row.  The 16-byte chunks of a staged row are
        // XOR-permuted by the row, so that the rows one fragment writes fall
        // in different bank groups.  (Blocks 16 wide along the contiguous
        // dimension gain nothing: their rows are 32-byte pieces anyway.)  The
        // write-back is a streaming (non-temporal) store: the kernel never
        // reads the output, and the operand panels keep the cache.
        constexpr int EA = 16 * kFA, EB = 16 * kFB;
        constexpr int W_STG = EA * EB * 2;             // staging bytes per wave
        constexpr int IN_B = 3 * kBStage / W_STG;      // waves staged in the B stages; the rest in the A stages
        static_assert(kWaves <= IN_B || (kWaves - IN_B) * W_STG <= 3 * kAStage, "staging fits the stages");
        constexpr int CPR_A = EA / 8, CPR_B = EB / 8;  // 16-byte chunks per staged row, along A or B
        constexpr int CPP_A = 64 / (CPR_A > 0 ? CPR_A : 1), CPP_B = 64 / (CPR_B > 0 ? CPR_B : 1);   // rows per read
        const int a_w = a0 + wa * EA, b_w = b0 + wb * EB;
        const bool along_a = kFA >= 2 && sya == 1 && (syb & 7) == 0;
        const bool along_b = kFB >= 2 && syb == 1 && (sya & 7) == 0;
        if ((along_a || along_b) && ((uintptr_t)Y & 15) == 0) {
            // every wave is done with the stages (its loads past the end have landed)
            __syncthreads();
            if (a_w + EA <= RA && b_w + EB <= RB) {
                uint8_t* stg = wave < IN_B ? bsb + wave * W_STG : asb + (wave - IN_B) * W_STG;
                uint16_t* const y = reinterpret_cast<uint16_t*>(Y);
                auto half16 = [](float f) { return OUT == SP24_BF16 ? f32_to_bf16_rne(f) : f32_to_f16_rne(f); };
                if constexpr (kFA >= 2) {
                    if (along_a) {
                        static_assert(CPR_A >= 4 && CPR_A <= 16 && EB % CPP_A == 0, "staged block shape");
                        // staged row bl (an output row): EA outputs, chunk c at slot c ^ sw(bl)
                        auto slot = [](int bl, int c) { return 16 * (c ^ ((bl / (16 / CPR_A)) & (CPR_A - 1))); };
#pragma unroll
                        for (int i = 0; i < kFA; ++i) {
#pragma unroll
                            for (int j = 0; j < kFB; ++j) {
                                const int al = i * 16 + 4 * kg, bl = j * 16 + r;
                                const f32x4 v = value(i, j, a_w + al, b_w + bl);
                                *reinterpret_cast<uint2*>(stg + bl * (EA * 2) + slot(bl, al >> 3) + 8 * ((al >> 2) & 1)) =
                                    make_uint2(half16(v[0]) | ((uint32_t)half16(v[1]) << 16),
                                               half16(v[2]) | ((uint32_t)half16(v[3]) << 16));
                            }
                        }
                        // this wave's LDS writes complete before it reads them back
                        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
                        __builtin_amdgcn_wave_barrier();
#pragma unroll
                        for (int pass = 0; pass < EB / CPP_A; ++pass) {
                            const int bl = pass * CPP_A + lane / CPR_A, c = lane % CPR_A;
                            const uint4 d = *reinterpret_cast<const uint4*>(stg + bl * (EA * 2) + slot(bl, c));
                            store_stream(y + (int64_t)(b_w + bl) * syb + a_w + 8 * c, d);
                        }
                        return;
                    }
                }
                if constexpr (kFB >= 2) {
                    if (along_b) {
                        static_assert(CPR_B >= 4 && CPR_B <= 16 && EA % CPP_B == 0, "staged block shape");
                        // staged row al (an output row): EB outputs, chunk c at slot c ^ sw(al)
                        auto slot = [](int al, int c) { return 16 * (c ^ ((al / (16 / CPR_B)) & (CPR_B - 1))); };
#pragma unroll
                        for (int i = 0; i < kFA; ++i) {
#pragma unroll
                            for (int j = 0; j < kFB; ++j) {
                                const int al = i * 16 + 4 * kg, bl = j * 16 + r;
                                const f32x4 v = value(i, j, a_w + al, b_w + bl);
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    *reinterpret_cast<uint16_t*>(stg + (al + q) * (EB * 2) + slot(al + q, bl >> 3) +
                                                                 2 * (bl & 7)) = half16(v[q]);
                            }
                        }
                        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
                        __builtin_amdgcn_wave_barrier();
#pragma unroll
                        for (int pass = 0; pass < EA / CPP_B; ++pass) {
                            const int al = pass * CPP_B + lane / CPR_B, c = lane % CPR_B;
                            const uint4 d = *reinterpret_cast<const uint4*>(stg + al * (EB * 2) + slot(al, c));
                            store_stream(y + (int64_t)(a_w + al) * sya + b_w + 8 * c, d);
                        }
                        return;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kFA; ++i) {
#pragma unroll
        for (int j = 0; j < kFB; ++j) {
            const int ar = a0 + wa * 16 * kFA + i * 16 + 4 * kg;
            const int br = b0 + wb * 16 * kFB + j * 16 + r;
            if (br >= RB || ar >= RA)
                continue;
            const f32x4 v = value(i, j, ar, br);
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

// Tile t (the workgroup's place in an XCD-aware order: consecutive t run on
// one XCD) -> (group, A tile, B tile), in groups of G A tiles x all B tiles.
struct TilePos {
    int group, ta, tb;
};
__device__ __forceinline__ int xcd_order_of(int b, int nwg) {
    const int xcd = b & 7, local = b >> 3;
    const int per_xcd = (nwg + 7) >> 3, full = nwg & 7 ? (nwg & 7) : 8;   // XCDs holding per_xcd tiles
    return xcd < full ? xcd * per_xcd + local : full * per_xcd + (xcd - full) * (per_xcd - 1) + local;
}
__device__ __forceinline__ int xcd_order(int nwg) { return xcd_order_of((int)blockIdx.x, nwg); }
__device__ __forceinline__ TilePos tile_pos(int t, int tiles_a, int tiles_b) {
    constexpr int G = 8;
    const int group = t / (G * tiles_b), within = t - group * G * tiles_b;
    const int g_rows = min(G, tiles_a - group * G);
    return {group, group * G + within % g_rows, within / g_rows};
}

#define SP24_TILE_LDS(TL)                                                                                    \
    __shared__ __attribute__((aligned(1024))) uint8_t asb[3 * TL::A_STAGE];                              \
    __shared__ __attribute__((aligned(1024))) uint8_t bsb[3 * TL::B_STAGE];                              \
    __shared__ __attribute__((aligned(1024))) uint8_t msb[kMetaSlots * TL::M_BLOCK]

template <sp24_dtype DT, sp24_dtype OUT, class TL>
__global__ void __launch_bounds__(TL::THREADS, TL::OCC)
sp24_big(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ B,
         const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ Y, int RA, int RB,
         int64_t K, int64_t sya, int64_t syb, int tiles_a, int tiles_b) {
    SP24_TILE_LDS(TL);
    const TilePos p = tile_pos(xcd_order(gridDim.x), tiles_a, tiles_b);
    tile_body<DT, OUT, TL, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, K,
                                  sya, syb, p.ta * TL::BA, p.tb * TL::BB, p.group);
}

// The 256 x 256 grid whose last round would leave most compute units idle:
// the first n_big tiles (whole rounds of the chip) run as in sp24_big; each
// later tile is split into `parts` smaller tiles -- four 128 x 128 quarters,
// or two 256 x 128 halves (along B) -- so that the remainder takes every
// compute unit for a shorter round instead of some of them for a full one.
// Each output element is still computed by exactly one workgroup.  The two
// ranges are ordered separately, so that the big tiles are dispatched first;
// the parts of a tile are consecutive in the XCD-aware order and share its
// operands through one XCD's L2.
template <sp24_dtype DT, sp24_dtype OUT>
__global__ void __launch_bounds__(T256x256::THREADS, 1)
sp24_big_tail(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ B,
              const float* __restrict__ sa, const float* __restrict__ sb, void* __restrict__ Y, int RA, int RB,
              int64_t K, int64_t sya, int64_t syb, int tiles_a, int tiles_b, int n_big, int parts) {
    static_assert(T128x128::THREADS == T256x256::THREADS && T256x128::THREADS == T256x256::THREADS,
                  "one block size");
    static_assert(T128x128::A_STAGE <= T256x256::A_STAGE && T128x128::B_STAGE <= T256x256::B_STAGE &&
                      T128x128::M_BLOCK <= T256x256::M_BLOCK, "the quarter tiles use the big tile's LDS");
    static_assert(T256x128::A_STAGE <= T256x256::A_STAGE && T256x128::B_STAGE <= T256x256::B_STAGE &&
                      T256x128::M_BLOCK <= T256x256::M_BLOCK, "the half tiles use the big tile's LDS");
    SP24_TILE_LDS(T256x256);
    const int b = (int)blockIdx.x;
    if (b < n_big) {
        const TilePos p = tile_pos(xcd_order_of(b, n_big), tiles_a, tiles_b);
        tile_body<DT, OUT, T256x256, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, K, sya, syb,
                                            p.ta * 256, p.tb * 256, p.group);
    } else if (parts == 2) {
        // n_big is a multiple of 8, so b - n_big keeps b's XCD
        const int q = xcd_order_of(b - n_big, (int)gridDim.x - n_big);
        const TilePos p = tile_pos(n_big + q / 2, tiles_a, tiles_b);
        tile_body<DT, OUT, T256x128, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, K, sya, syb,
                                            p.ta * 256, p.tb * 256 + 128 * (q & 1), p.group);
    } else {
        // n_big is a multiple of 8, so b - n_big keeps b's XCD
        const int q = xcd_order_of(b - n_big, (int)gridDim.x - n_big);
        const TilePos p = tile_pos(n_big + q / 4, tiles_a, tiles_b);
        tile_body<DT, OUT, T128x128, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, K, sya, syb,
                                            p.ta * 256 + 128 * ((q >> 1) & 1), p.tb * 256 + 128 * (q & 1), p.group);
    }
}

// The hybrid GEMM in one launch: the first tiles_s * tiles_b workgroups (in
// the XCD-aware order) take the compressed rows [0, RS) of A, the rest the
// dense rows [0, RD) of Ad, whose outputs start at Yd (scales at sd); both
// share B, its scales and the output strides.
template <sp24_dtype DT, sp24_dtype OUT, class TL>
__global__ void __launch_bounds__(TL::THREADS, TL::OCC)
sp24_hybrid(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ ad,
            const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sd,
            const float* __restrict__ sb, void* __restrict__ Y, void* __restrict__ Yd, int RS, int RD, int RB,
            int64_t K, int64_t sya, int64_t syb, int tiles_s, int tiles_d, int tiles_b) {
    SP24_TILE_LDS(TL);
    const int t = xcd_order(gridDim.x);
    if (t < tiles_s * tiles_b) {
        const TilePos p = tile_pos(t, tiles_s, tiles_b);
        tile_body<DT, OUT, TL, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RS, RB, K,
                                      sya, syb, p.ta * TL::BA, p.tb * TL::BB, p.group);
    } else {
        const TilePos p = tile_pos(t - tiles_s * tiles_b, tiles_d, tiles_b);
        tile_body<DT, OUT, TL, true>(asb, bsb, msb, ad, nullptr, B, sd, sb, Yd, RD,
                                     RB, K, sya, syb, p.ta * (TL::BA / 2), p.tb * TL::BB, p.group);
    }
}

// The hybrid grid with a short last round, split as sp24_big_tail splits the
// plain one: the first n_big tiles (compressed, then dense, as in
// sp24_hybrid) whole, each later one as four quarter tiles of its region
// (a dense quarter: 64 dense rows x 128 rows of B).
template <sp24_dtype DT, sp24_dtype OUT>
__global__ void __launch_bounds__(T256x256::THREADS, 1)
sp24_hybrid_tail(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ ad,
                 const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sd,
                 const float* __restrict__ sb, void* __restrict__ Y, void* __restrict__ Yd, int RS, int RD, int RB,
                 int64_t K, int64_t sya, int64_t syb, int tiles_s, int tiles_d, int tiles_b, int n_big) {
    SP24_TILE_LDS(T256x256);
    const int b = (int)blockIdx.x, ns = tiles_s * tiles_b;
    int t = 0, q = -1;   // tile, and the quarter of it (-1: whole)
    if (b < n_big) {
        t = xcd_order_of(b, n_big);
    } else {
        // n_big is a multiple of 8, so b - n_big keeps b's XCD
        const int qq = xcd_order_of(b - n_big, (int)gridDim.x - n_big);
        t = n_big + qq / 4;
        q = qq & 3;
    }
    const int qa = (q >> 1) & 1, qb = q & 1;
    if (t < ns) {
        const TilePos p = tile_pos(t, tiles_s, tiles_b);
        if (q < 0)
            tile_body<DT, OUT, T256x256, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RS, RB, K, sya, syb,
                                                p.ta * 256, p.tb * 256, p.group);
        else
            tile_body<DT, OUT, T128x128, false>(asb, bsb, msb, av, am, B, sa, sb, Y, RS, RB, K, sya, syb,
                                                p.ta * 256 + 128 * qa, p.tb * 256 + 128 * qb, p.group);
    } else {
        const TilePos p = tile_pos(t - ns, tiles_d, tiles_b);
        if (q < 0)
            tile_body<DT, OUT, T256x256, true>(asb, bsb, msb, ad, nullptr, B, sd, sb, Yd, RD, RB, K, sya, syb,
                                               p.ta * 128, p.tb * 256, p.group);
        else
            tile_body<DT, OUT, T128x128, true>(asb, bsb, msb, ad, nullptr, B, sd, sb, Yd, RD, RB, K, sya, syb,
                                               p.ta * 128 + 64 * qa, p.tb * 256 + 128 * qb, p.group);
    }
}

// The K-split hybrid GEMM: every tile runs the compressed K range of its
// weight rows and then their dense K range, into one set of accumulators
// (tile_body's KSPLIT form).  A = W (rows RA = N), B = X (rows RB = M).
template <sp24_dtype DT, sp24_dtype OUT, class TL>
__global__ void __launch_bounds__(TL::THREADS, TL::OCC)
sp24_ksplit(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ ad,
            const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
            void* __restrict__ Y, int RA, int RB, int64_t KS, int64_t KD, int64_t sya, int64_t syb, int tiles_a,
            int tiles_b) {
    SP24_TILE_LDS(TL);
    const TilePos p = tile_pos(xcd_order(gridDim.x), tiles_a, tiles_b);
    tile_body<DT, OUT, TL, false, true>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, KS, sya, syb,
                                        p.ta * TL::BA, p.tb * TL::BB, p.group, ad, KD);
}

// The K-split grid with a short last round, split into quarter or half tiles
// as sp24_big_tail splits the plain one.
template <sp24_dtype DT, sp24_dtype OUT>
__global__ void __launch_bounds__(T256x256::THREADS, 1)
sp24_ksplit_tail(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am, const uint8_t* __restrict__ ad,
                 const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
                 void* __restrict__ Y, int RA, int RB, int64_t KS, int64_t KD, int64_t sya, int64_t syb,
                 int tiles_a, int tiles_b, int n_big, int parts) {
    SP24_TILE_LDS(T256x256);
    const int b = (int)blockIdx.x;
    if (b < n_big) {
        const TilePos p = tile_pos(xcd_order_of(b, n_big), tiles_a, tiles_b);
        tile_body<DT, OUT, T256x256, false, true>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, KS, sya, syb,
                                                  p.ta * 256, p.tb * 256, p.group, ad, KD);
    } else if (parts == 2) {
        const int q = xcd_order_of(b - n_big, (int)gridDim.x - n_big);
        const TilePos p = tile_pos(n_big + q / 2, tiles_a, tiles_b);
        tile_body<DT, OUT, T256x128, false, true>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, KS, sya, syb,
                                                  p.ta * 256, p.tb * 256 + 128 * (q & 1), p.group, ad, KD);
    } else {
        const int q = xcd_order_of(b - n_big, (int)gridDim.x - n_big);
        const TilePos p = tile_pos(n_big + q / 4, tiles_a, tiles_b);
        tile_body<DT, OUT, T128x128, false, true>(asb, bsb, msb, av, am, B, sa, sb, Y, RA, RB, KS, sya, syb,
                                                  p.ta * 256 + 128 * ((q >> 1) & 1), p.tb * 256 + 128 * (q & 1),
                                                  p.group, ad, KD);
    }
}

template <sp24_dtype DT, sp24_dtype OUT, class TL>
hipError_t launch_tile(const GemmArgs& g, hipStream_t s, const char** kname, const char* name) {
    const int RA = (int)(g.a_is_w ? g.N : g.M);
    const int RB = (int)(g.a_is_w ? g.M : g.N);
    const int64_t sya = g.a_is_w ? 1 : g.N, syb = g.a_is_w ? g.N : 1;
    const int tiles_a = (RA + TL::BA - 1) / TL::BA, tiles_b = (RB + TL::BB - 1) / TL::BB;
    if (kname)
        *kname = name;
    if (g.dry)
        return hipSuccess;
    hipLaunchKernelGGL((sp24_big<DT, OUT, TL>), dim3(tiles_a * tiles_b), dim3(TL::THREADS), 0, s,
                       (const uint8_t*)g.a_vals, g.a_meta, (const uint8_t*)g.b, g.scale_a, g.scale_b, g.Y, RA,
                       RB, g.K, sya, syb, tiles_a, tiles_b);
    return hipGetLastError();
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_tail(const GemmArgs& g, hipStream_t s, const char** kname, int64_t n_big, int64_t n_split,
                       int parts) {
    const int RA = (int)(g.a_is_w ? g.N : g.M);
    const int RB = (int)(g.a_is_w ? g.M : g.N);
    const int64_t sya = g.a_is_w ? 1 : g.N, syb = g.a_is_w ? g.N : 1;
    const int tiles_a = (RA + 255) / 256, tiles_b = (RB + 255) / 256;
    if (kname)
        *kname = "sp24_big_256x256_tail";
    if (g.dry)
        return hipSuccess;
    hipLaunchKernelGGL((sp24_big_tail<DT, OUT>), dim3((unsigned)(n_big + parts * n_split)), dim3(T256x256::THREADS),
                       0, s, (const uint8_t*)g.a_vals, g.a_meta, (const uint8_t*)g.b, g.scale_a, g.scale_b, g.Y, RA,
                       RB, g.K, sya, syb, tiles_a, tiles_b, (int)n_big, parts);
    return hipGetLastError();
}

// Between 256 x 256 and 256 x 128 tiles when the big ones alone would not
// fill the chip: the one whose rounds cost less, a round of 256 x 128 tiles
// counted as 0.7 of a round of 256 x 256 ones (measured 0.66-0.75 on the
// bf16 prefill shapes).  So a 256 x 256 grid of one round beats a 256 x 128
// grid of two.
inline bool prefer_256(int64_t t256, int64_t t128, int64_t cus) {
    const int64_t r256 = (t256 + cus - 1) / cus, r128 = (t128 + cus - 1) / cus;
    return 10 * r256 <= 7 * r128;
}

template <class TL>
int64_t tiles_rc(int64_t RA, int64_t RB) {
    return ((RA + TL::BA - 1) / TL::BA) * ((RB + TL::BB - 1) / TL::BB) * TL::OCC;
}

// Which tile grid runs an RA x RB output.
enum TileKind { kT256, kT256Tail, kT256x128, kT128x128, kT128x64, kT256x64 };
struct TilePlan {
    TileKind kind;
    int64_t n_big, n_split;   // kT256Tail: whole 256 x 256 tiles, and the tiles split into parts
    int parts;                // kT256Tail: 4 (128 x 128 quarters) or 2 (256 x 128 halves)
};

// The largest tile that keeps most CUs busy (measured: 256 x 256 from 192
// tiles on); failing that, the smallest.  The smaller tiles run two
// workgroups per CU.  A 256 x 256 grid of more than one round whose last
// round would fill at most a quarter of the chip runs that round as quarter
// tiles (sp24_big_tail); with `halves`, one that would fill at most half of
// it runs as half tiles.
inline TilePlan plan_tiles(int64_t RA, int64_t RB, bool halves = false) {
    constexpr int64_t kFill = 192;
    constexpr int64_t kCUs = 256;   // compute units of the gfx950 parts (MI350X, MI355X)
    if (RB > 64) {
        const int64_t t256 = tiles_rc<T256x256>(RA, RB), rest = t256 % kCUs;
        // past one round: a remainder whose quarters fill at most one round goes
        // to quarter tiles (measured: 20-32% faster at remainders of 16 and 64
        // tiles; at 128, two rounds of quarters, -1% bf16 to +2.5% fp8)
        if (t256 > kCUs && rest > 0 && 4 * rest <= kCUs) return {kT256Tail, t256 - rest, rest, 4};
        if (halves && t256 > kCUs && rest > 0 && 2 * rest <= kCUs) return {kT256Tail, t256 - rest, rest, 2};
        const int64_t t128 = tiles_rc<T256x128>(RA, RB);
        if (t256 >= kFill || (t128 >= kFill && prefer_256(t256, t128, kCUs))) return {kT256, 0, 0};
        if (t128 >= kFill) return {kT256x128, 0, 0};
        // 128 x 128 tiles while they alone keep most CUs busy; fewer, the
        // 128 x 64 ones (measured: 14-19% faster at 128 tiles of 128 x 128)
        if (tiles_rc<T128x128>(RA, RB) / T128x128::OCC >= kFill) return {kT128x128, 0, 0};
        return {kT128x64, 0, 0};
    }
    if (tiles_rc<T256x64>(RA, RB) >= kFill) return {kT256x64, 0, 0};
    return {kT128x64, 0, 0};
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_big(const GemmArgs& g, hipStream_t s, const char** kname) {
    const int64_t RA = g.a_is_w ? g.N : g.M, RB = g.a_is_w ? g.M : g.N;
    const TilePlan p = plan_tiles(RA, RB, true);
    switch (p.kind) {
    case kT256Tail: return launch_tail<DT, OUT>(g, s, kname, p.n_big, p.n_split, p.parts);
    case kT256: return launch_tile<DT, OUT, T256x256>(g, s, kname, "sp24_big_256x256");
    case kT256x128: return launch_tile<DT, OUT, T256x128>(g, s, kname, "sp24_big_256x128");
    case kT128x128: return launch_tile<DT, OUT, T128x128>(g, s, kname, "sp24_big_128x128");
    case kT256x64: return launch_tile<DT, OUT, T256x64>(g, s, kname, "sp24_big_256x64");
    default: return launch_tile<DT, OUT, T128x64>(g, s, kname, "sp24_big_128x64");
    }
}

template <sp24_dtype DT, sp24_dtype OUT, class TL>
hipError_t launch_ksplit_tile(const KsplitArgs& k, hipStream_t s, const char** kname, const char* name) {
    const int RA = (int)k.N, RB = (int)k.M;
    const int tiles_a = (RA + TL::BA - 1) / TL::BA, tiles_b = (RB + TL::BB - 1) / TL::BB;
    if (kname)
        *kname = name;
    if (k.dry)
        return hipSuccess;
    hipLaunchKernelGGL((sp24_ksplit<DT, OUT, TL>), dim3(tiles_a * tiles_b), dim3(TL::THREADS), 0, s,
                       (const uint8_t*)k.ws_vals, k.ws_meta, (const uint8_t*)k.wd, (const uint8_t*)k.x, k.scale_w,
                       k.scale_x, k.Y, RA, RB, k.KS, k.K - k.KS, (int64_t)1, k.N, tiles_a, tiles_b);
    return hipGetLastError();
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_ksplit_tiles(const KsplitArgs& k, hipStream_t s, const char** kname) {
    const TilePlan p = plan_tiles(k.N, k.M, true);
    switch (p.kind) {
    case kT256Tail: {
        const int RA = (int)k.N, RB = (int)k.M;
        if (kname)
            *kname = "sp24_ksplit_256x256_tail";
        if (k.dry)
            return hipSuccess;
        hipLaunchKernelGGL((sp24_ksplit_tail<DT, OUT>), dim3((unsigned)(p.n_big + p.parts * p.n_split)),
                           dim3(T256x256::THREADS), 0, s, (const uint8_t*)k.ws_vals, k.ws_meta,
                           (const uint8_t*)k.wd, (const uint8_t*)k.x, k.scale_w, k.scale_x, k.Y, RA, RB, k.KS,
                           k.K - k.KS, (int64_t)1, k.N, (RA + 255) / 256, (RB + 255) / 256, (int)p.n_big, p.parts);
        return hipGetLastError();
    }
    case kT256: return launch_ksplit_tile<DT, OUT, T256x256>(k, s, kname, "sp24_ksplit_256x256");
    case kT256x128: return launch_ksplit_tile<DT, OUT, T256x128>(k, s, kname, "sp24_ksplit_256x128");
    case kT128x128: return launch_ksplit_tile<DT, OUT, T128x128>(k, s, kname, "sp24_ksplit_128x128");
    case kT256x64: return launch_ksplit_tile<DT, OUT, T256x64>(k, s, kname, "sp24_ksplit_256x64");
    default: return launch_ksplit_tile<DT, OUT, T128x64>(k, s, kname, "sp24_ksplit_128x64");
    }
}

template <sp24_dtype DT, sp24_dtype OUT, class TL>
hipError_t launch_hybrid_tile(const HybridArgs& h, hipStream_t s, const char** kname, const char* name) {
    const int RS = (int)h.NS, RD = (int)h.ND, RB = (int)h.M;
    const int tiles_s = (RS + TL::BA - 1) / TL::BA, tiles_d = (RD + TL::BA / 2 - 1) / (TL::BA / 2);
    const int tiles_b = (RB + TL::BB - 1) / TL::BB;
    if (kname)
        *kname = name;
    if (h.dry)
        return hipSuccess;
    void* Yd = (uint8_t*)h.Y + h.NS * elem_bytes(OUT);
    hipLaunchKernelGGL((sp24_hybrid<DT, OUT, TL>), dim3((tiles_s + tiles_d) * tiles_b), dim3(TL::THREADS), 0, s,
                       (const uint8_t*)h.ws_vals, h.ws_meta, (const uint8_t*)h.wd, (const uint8_t*)h.x, h.scale_w,
                       h.scale_w ? h.scale_w + h.NS : nullptr, h.scale_x, h.Y, Yd, RS, RD, RB, h.K, (int64_t)1,
                       h.NS + h.ND, tiles_s, tiles_d, tiles_b);
    return hipGetLastError();
}

template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_hybrid_tail(const HybridArgs& h, hipStream_t s, const char** kname, int64_t n_big,
                              int64_t n_split) {
    const int RS = (int)h.NS, RD = (int)h.ND, RB = (int)h.M;
    const int tiles_s = (RS + 255) / 256, tiles_d = (RD + 127) / 128, tiles_b = (RB + 255) / 256;
    if (kname)
        *kname = "sp24_hybrid_256x256_tail";
    if (h.dry)
        return hipSuccess;
    void* Yd = (uint8_t*)h.Y + h.NS * elem_bytes(OUT);
    hipLaunchKernelGGL((sp24_hybrid_tail<DT, OUT>), dim3((unsigned)(n_big + 4 * n_split)), dim3(T256x256::THREADS), 0,
                       s, (const uint8_t*)h.ws_vals, h.ws_meta, (const uint8_t*)h.wd, (const uint8_t*)h.x, h.scale_w,
                       h.scale_w ? h.scale_w + h.NS : nullptr, h.scale_x, h.Y, Yd, RS, RD, RB, h.K, (int64_t)1,
                       h.NS + h.ND, tiles_s, tiles_d, tiles_b, (int)n_big);
    return hipGetLastError();
}

template <class TL>
int64_t hybrid_tiles_of(const HybridArgs& h) {
    const int64_t ts = (h.NS + TL::BA - 1) / TL::BA, td = (h.ND + TL::BA / 2 - 1) / (TL::BA / 2);
    return (ts + td) * ((h.M + TL::BB - 1) / TL::BB) * TL::OCC;
}

// The tile choice of the plain GEMM, counting the dense region's half-height tiles.
template <sp24_dtype DT, sp24_dtype OUT>
hipError_t launch_hybrid(const HybridArgs& h, hipStream_t s, const char** kname) {
    constexpr int64_t kFill = 192;
    constexpr int64_t kCUs = 256;
    if (h.M > 64) {
        const int64_t t256 = hybrid_tiles_of<T256x256>(h), t128 = hybrid_tiles_of<T256x128>(h);
        const int64_t rest = t256 % kCUs;
        if (t256 > kCUs && rest > 0 && 4 * rest <= kCUs)
            return launch_hybrid_tail<DT, OUT>(h, s, kname, t256 - rest, rest);
        if (t256 >= kFill || (t128 >= kFill && prefer_256(t256, t128, kCUs)))
            return launch_hybrid_tile<DT, OUT, T256x256>(h, s, kname, "sp24_hybrid_256x256");
        if (t128 >= kFill)
            return launch_hybrid_tile<DT, OUT, T256x128>(h, s, kname, "sp24_hybrid_256x128");
        if (hybrid_tiles_of<T128x128>(h) / T128x128::OCC >= kFill)
            return launch_hybrid_tile<DT, OUT, T128x128>(h, s, kname, "sp24_hybrid_128x128");
        return launch_hybrid_tile<DT, OUT, T128x64>(h, s, kname, "sp24_hybrid_128x64");
    }
    if (hybrid_tiles_of<T256x64>(h) >= kFill)
        return launch_hybrid_tile<DT, OUT, T256x64>(h, s, kname, "sp24_hybrid_256x64");
    return launch_hybrid_tile<DT, OUT, T128x64>(h, s, kname, "sp24_hybrid_128x64");
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
    case SP24_I8:
        if (g.out_dt == SP24_BF16) return launch_big<SP24_I8, SP24_BF16>(g, s, kname);
        return launch_big<SP24_I8, SP24_F32>(g, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_sp24_ksplit(const KsplitArgs& k, hipStream_t s, const char** kname) {
    switch (k.in_dt) {
    case SP24_BF16:
        if (k.out_dt == SP24_BF16) return launch_ksplit_tiles<SP24_BF16, SP24_BF16>(k, s, kname);
        if (k.out_dt == SP24_F16) return launch_ksplit_tiles<SP24_BF16, SP24_F16>(k, s, kname);
        return launch_ksplit_tiles<SP24_BF16, SP24_F32>(k, s, kname);
    case SP24_F16:
        if (k.out_dt == SP24_F16) return launch_ksplit_tiles<SP24_F16, SP24_F16>(k, s, kname);
        if (k.out_dt == SP24_BF16) return launch_ksplit_tiles<SP24_F16, SP24_BF16>(k, s, kname);
        return launch_ksplit_tiles<SP24_F16, SP24_F32>(k, s, kname);
    case SP24_E4M3:
        if (k.out_dt == SP24_BF16) return launch_ksplit_tiles<SP24_E4M3, SP24_BF16>(k, s, kname);
        return launch_ksplit_tiles<SP24_E4M3, SP24_F32>(k, s, kname);
    case SP24_I8:
        if (k.out_dt == SP24_BF16) return launch_ksplit_tiles<SP24_I8, SP24_BF16>(k, s, kname);
        return launch_ksplit_tiles<SP24_I8, SP24_F32>(k, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

hipError_t launch_sp24_hybrid(const HybridArgs& h, hipStream_t s, const char** kname) {
    switch (h.in_dt) {
    case SP24_BF16:
        if (h.out_dt == SP24_BF16) return launch_hybrid<SP24_BF16, SP24_BF16>(h, s, kname);
        if (h.out_dt == SP24_F16) return launch_hybrid<SP24_BF16, SP24_F16>(h, s, kname);
        return launch_hybrid<SP24_BF16, SP24_F32>(h, s, kname);
    case SP24_F16:
        if (h.out_dt == SP24_F16) return launch_hybrid<SP24_F16, SP24_F16>(h, s, kname);
        if (h.out_dt == SP24_BF16) return launch_hybrid<SP24_F16, SP24_BF16>(h, s, kname);
        return launch_hybrid<SP24_F16, SP24_F32>(h, s, kname);
    case SP24_E4M3:
        if (h.out_dt == SP24_BF16) return launch_hybrid<SP24_E4M3, SP24_BF16>(h, s, kname);
        return launch_hybrid<SP24_E4M3, SP24_F32>(h, s, kname);
    case SP24_I8:
        if (h.out_dt == SP24_BF16) return launch_hybrid<SP24_I8, SP24_BF16>(h, s, kname);
        return launch_hybrid<SP24_I8, SP24_F32>(h, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
