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
// The decode kernel and the dispatch of every sparse GEMM:
//   skinny  few B rows (decode: M <= 64).  HBM-bound on the compressed
//           weight.  One workgroup owns 16 (or 32) rows of A and all of B;
//           its waves split K into runs of 8-step groups, issue every load
//           of a group at once (A into registers, metadata and up to 4 B rows
//           into LDS by direct global->LDS loads), and reduce their partial
//           tiles through LDS in a fixed order (deterministic, no atomics).
//           5 to 16 B rows: sp24_skinny_x16, the same with all 16 rows staged.
// Larger B goes to the LDS-staged tile kernels of gemm_sparse_big.hip.
#include "mfma_ops.h"

namespace sp24 {
namespace {

// ------------------------------------------------------------------ skinny
constexpr int kMaxWaves = 8;
constexpr int kGroup = 8;   // K-steps per load group

typedef __attribute__((address_space(3))) void lds_void;

// Per wave and load group: the group's metadata of the 16 * AT rows (1 KiB
// per 16 rows for 16-bit steps, 2 KiB for fp8) and, for at most 4 dense rows,
// the group's slice of those rows (4 x 1 KiB) plus a zero pad read by the
// empty lanes.
template <int MWS, int AT>
struct SkinnyLds {
    static constexpr int META = 16 * AT * kGroup * MWS * 4;
    static constexpr int XROWS = 4;
    static constexpr int X = XROWS * kGroup * 128;
    static constexpr int PER_WAVE = META + X + 32;
};

// AT: 16-row A tiles per workgroup (2 halves the B traffic per A byte when
// there are enough tiles to fill the chip); MT: 16-column B fragments held in
// registers at once; PASSES: passes over the group with MT fragments each
// (the A registers are reused; B in registers for a whole group costs
// 8 steps x MT x 32 bytes per lane).
template <sp24_dtype DT, sp24_dtype OUT, int MT, bool XLDS, int AT, int PASSES>
__global__ void __launch_bounds__(kMaxWaves * 64, 2)
sp24_skinny(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am,
            const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
            void* __restrict__ Y, int RA, int RB, int64_t K, int64_t sya, int64_t syb) {
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    constexpr int MWS = L::META_WORDS;
    using SL = SkinnyLds<MWS, AT>;
    constexpr int M_ROW = kGroup * MWS * 4;         // metadata bytes of one row per group: 64 or 128
    constexpr int M_CPR = M_ROW / 16;               // 16-byte chunks per row: 4 or 8
    constexpr int M_LOADS = SL::META / 1024;        // AT or 2 * AT
    constexpr int M_RPL = 1024 / M_ROW;             // rows per load: 16 or 8
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kMaxWaves][SL::PER_WAVE];
    constexpr int MTT = MT * PASSES;                // B fragments in all
    __shared__ float red[kMaxWaves][AT][MTT][4][64];

    const int WAVES = blockDim.x >> 6;   // the waves split K
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, kg = lane >> 4;
    const int a0 = blockIdx.x * 16 * AT;
    const int steps = (int)(K / L::KSTEP);
    const int groups = (steps + kGroup - 1) / kGroup;
    const uint32_t a_row_bytes = (uint32_t)(K / 2 * L::ELEM), b_row_bytes = (uint32_t)(K * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);   // rows past RA / RB read as zeros
    const Buf bufM(am, (uint32_t)RA * m_row_bytes);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);
    uint8_t* my_m = &lds[wave][0];
    uint8_t* my_x = &lds[wave][SL::META];
    uint8_t* zero_pad = &lds[wave][SL::META + SL::X];
    if (XLDS && lane < 8)
        reinterpret_cast<uint32_t*>(zero_pad)[lane] = 0u;

    // A: straight from HBM into the operand registers, one 1 KiB load per step and tile
    uint32_t a_base[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
        a_base[t] = (uint32_t)(a0 + 16 * t + r) * a_row_bytes + L::a_off(kg);
    // metadata: DMA lane roles (row, chunk slot), chunks XOR-swizzled by row
    const int m_swz_r = M_CPR == 4 ? (r >> 2) & 3 : (r >> 1) & 7;
    const int msh = L::meta_shift(kg), mwd = L::meta_word(kg);
    // X through registers (more than 4 dense rows) or through LDS (at most 4)
    uint32_t b_base[MTT];
#pragma unroll
    for (int mt = 0; mt < MTT; ++mt)
        b_base[mt] = (uint32_t)(mt * 16 + r) * b_row_bytes;

    f32x4 acc[AT][MTT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int mt = 0; mt < MTT; ++mt)
            acc[t][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // each wave streams a contiguous run of groups; the run of the whole
    // workgroup starts at a rotated group so that concurrent workgroups read
    // different column offsets of their (power-of-two strided) rows
    const int per_wave = (groups + WAVES - 1) / WAVES;
    const int rot = (int)((blockIdx.x * 5u) % (unsigned)max(groups, 1));
    for (int gi = 0; gi < per_wave; ++gi) {
        const int gl = wave * per_wave + gi;
        if (gl >= groups)
            break;
        const int g = gl + rot >= groups ? gl + rot - groups : gl + rot;
        const int s_first = g * kGroup;
        const int n_in = min(kGroup, steps - s_first);
        // ---- issue: A for the group's steps, metadata and X by DMA
        uint4 fa[AT][kGroup];
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                fa[t][u] = bufA.ld16(u < n_in ? a_base[t] + (uint32_t)(s_first + u) * L::A_STEP_BYTES : kOOB);
#pragma unroll
        for (int h = 0; h < M_LOADS; ++h) {
            const int row = h * M_RPL + lane / M_CPR;
            const int swz = M_CPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
            const uint32_t col = (uint32_t)g * M_ROW + 16 * ((lane % M_CPR) ^ swz);
            const bool in = col < m_row_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bufM.r, (lds_void*)(my_m + 1024 * h), 16,
                                                     (int)(in ? (uint32_t)(a0 + row) * m_row_bytes + col : kOOB),
                                                     0, 0, 0);
        }
        if (XLDS) {
#pragma unroll
            for (int j = 0; j < SL::XROWS; ++j) {
                if (j >= RB)
                    break;
                const uint32_t col = (uint32_t)s_first * L::B_STEP_BYTES + 16 * lane;
                const bool in = col < b_row_bytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(bufB.r, (lds_void*)(my_x + 1024 * j), 16,
                                                         (int)(in ? (uint32_t)j * b_row_bytes + col : kOOB), 0, 0, 0);
            }
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            uint4 xb0[kGroup][MT], xb1[kGroup][MT];
            if (!XLDS) {
#pragma unroll
                for (int u = 0; u < kGroup; ++u)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const uint32_t o = u < n_in ? b_base[p * MT + mt] + (uint32_t)(s_first + u) * L::B_STEP_BYTES
                                                    : kOOB;
                        xb0[u][mt] = bufB.ld16(o + L::b_off0(kg));
                        xb1[u][mt] = bufB.ld16(o + L::b_off1(kg));
                    }
            }
            // ---- the pass's loads (this wave's only) have landed
            __builtin_amdgcn_s_waitcnt((0) | (0x7 << 4) | (0xF << 8));
            // steps past the end of K (last group only) were loaded as zeros
            // and add nothing; running them keeps every load of the group used
            // unconditionally, which keeps the compiler from sinking each load
            // next to its use (one memory round trip per step)
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int wbyte = 4 * (MWS * u + mwd);
                uint32_t idx[AT];
#pragma unroll
                for (int t = 0; t < AT; ++t)
                    idx[t] = *reinterpret_cast<const uint32_t*>(my_m + M_ROW * (16 * t + r) +
                                                                16 * ((wbyte >> 4) ^ m_swz_r) + (wbyte & 15)) >> msh;
                if (XLDS) {
                    const uint8_t* xr = r < RB ? my_x + 1024 * r + 128 * u : zero_pad;
                    const int o0 = r < RB ? L::b_off0(kg) : 0, o1 = r < RB ? L::b_off1(kg) : 0;
                    const uint4 b0 = *reinterpret_cast<const uint4*>(xr + o0);
                    const uint4 b1 = *reinterpret_cast<const uint4*>(xr + o1);
#pragma unroll
                    for (int t = 0; t < AT; ++t)
                        acc[t][0] = Op::mma(fa[t][u], b0, b1, idx[t], acc[t][0]);
                } else {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int t = 0; t < AT; ++t)
                            acc[t][p * MT + mt] = Op::mma(fa[t][u], xb0[u][mt], xb1[u][mt], idx[t], acc[t][p * MT + mt]);
                }
            }
        }
        // the next group's DMA reuses this wave's LDS: finish reading it
        __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
    }

#pragma unroll
    for (int t = 0; t < AT; ++t)
#pragma unroll
        for (int mt = 0; mt < MTT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[wave][t][mt][i][lane] = acc[t][mt][i];
    __syncthreads();

    // D[4*kg + i][l % 16] of fragment (t, mt) lives at red[.][t][mt][i][kg*16 + l%16]
    constexpr int TILE = 16 * 16 * MTT;
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
        const int ar = a0 + 16 * t + al, br = bl;
        if (ar < RA && br < RB) {
            if (sa)
                v *= sa[ar];
            if (sb)
                v *= sb[br];
            store_out<OUT>(Y, (int64_t)ar * sya + (int64_t)br * syb, v);
        }
    }
}

// 5 to 16 dense rows: the plan above with all 16 rows of B staged in LDS.
// In registers, a B fragment puts 16 different rows in every 16 lanes, so
// each lane's 16 bytes is a request of its own to L2; staged, each row of the
// group is one contiguous 1 KiB load (8 whole lines).  The 16-byte chunks of
// a staged row are XOR-permuted by the row number, so that the 16 rows read
// by one fragment load fall in 16 different bank groups.  After the K loop
// the staging area holds the cross-wave reduction.  WV: waves per workgroup.
template <sp24_dtype DT, sp24_dtype OUT, int AT, int WV>
__global__ void __launch_bounds__(WV * 64)
sp24_skinny_x16(const uint8_t* __restrict__ av, const uint32_t* __restrict__ am,
                const uint8_t* __restrict__ B, const float* __restrict__ sa, const float* __restrict__ sb,
                void* __restrict__ Y, int RA, int RB, int64_t K, int64_t sya, int64_t syb) {
    using L = StepLayout<DT>;
    using Op = SparseOp<DT>;
    constexpr int MWS = L::META_WORDS;
    constexpr int M_ROW = kGroup * MWS * 4;         // metadata bytes of one row per group: 64 or 128
    constexpr int M_CPR = M_ROW / 16;               // 16-byte chunks per row: 4 or 8
    constexpr int META = 16 * AT * M_ROW;           // metadata of the group's 16 * AT rows
    constexpr int M_LOADS = META / 1024;
    constexpr int M_RPL = 1024 / M_ROW;             // rows per load: 16 or 8
    constexpr int X_ROW = kGroup * L::B_STEP_BYTES; // one B row of the group
    static_assert(X_ROW == 1024, "one 1 KiB load per staged row and group");
    constexpr int PER_WAVE = META + 16 * X_ROW;
    static_assert(AT * 4 * 64 * 4 <= PER_WAVE, "the reduction fits in the staging area");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[WV * PER_WAVE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, kg = lane >> 4;
    const int a0 = blockIdx.x * 16 * AT;
    const int steps = (int)(K / L::KSTEP);
    const int groups = (steps + kGroup - 1) / kGroup;
    const uint32_t a_row_bytes = (uint32_t)(K / 2 * L::ELEM), b_row_bytes = (uint32_t)(K * L::ELEM);
    const uint32_t m_row_bytes = (uint32_t)(K / 8);
    const Buf bufA(av, (uint32_t)RA * a_row_bytes);   // rows past RA / RB read as zeros
    const Buf bufM(am, (uint32_t)RA * m_row_bytes);
    const Buf bufB(B, (uint32_t)RB * b_row_bytes);
    uint8_t* my_m = lds + wave * PER_WAVE;
    uint8_t* my_x = my_m + META;

    uint32_t a_base[AT];
#pragma unroll
    for (int t = 0; t < AT; ++t)
        a_base[t] = (uint32_t)(a0 + 16 * t + r) * a_row_bytes + L::a_off(kg);
    const int m_swz_r = M_CPR == 4 ? (r >> 2) & 3 : (r >> 1) & 7;
    const int msh = L::meta_shift(kg), mwd = L::meta_word(kg);
    // this lane's B row in LDS and its two chunks of step 0 (before the permutation)
    const uint8_t* xr = my_x + X_ROW * r;
    const int xc0 = L::b_off0(kg) / 16, xc1 = L::b_off1(kg) / 16;

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
        const int s_first = g * kGroup;
        const int n_in = min(kGroup, steps - s_first);
        uint4 fa[AT][kGroup];
#pragma unroll
        for (int t = 0; t < AT; ++t)
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                fa[t][u] = bufA.ld16(u < n_in ? a_base[t] + (uint32_t)(s_first + u) * L::A_STEP_BYTES : kOOB);
#pragma unroll
        for (int h = 0; h < M_LOADS; ++h) {
            const int row = h * M_RPL + lane / M_CPR;
            const int swz = M_CPR == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
            const uint32_t col = (uint32_t)g * M_ROW + 16 * ((lane % M_CPR) ^ swz);
            const bool in = col < m_row_bytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bufM.r, (lds_void*)(my_m + 1024 * h), 16,
                                                     (int)(in ? (uint32_t)(a0 + row) * m_row_bytes + col : kOOB),
                                                     0, 0, 0);
        }
        // B row j: lane l fetches the chunk that belongs in slot l, chunk l ^ j
        // (rows past RB and steps past K load zeros)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t col = (uint32_t)s_first * L::B_STEP_BYTES + 16 * (lane ^ j);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bufB.r, (lds_void*)(my_x + X_ROW * j), 16,
                                                     (int)(col < b_row_bytes ? (uint32_t)j * b_row_bytes + col : kOOB),
                                                     0, 0, 0);
        }
        // this wave's loads have landed
        __builtin_amdgcn_s_waitcnt((0) | (0x7 << 4) | (0xF << 8));
        // steps past the end of K run on zeros (see sp24_skinny)
#pragma unroll
        for (int u = 0; u < kGroup; ++u) {
            const int wbyte = 4 * (MWS * u + mwd);
            uint32_t idx[AT];
#pragma unroll
            for (int t = 0; t < AT; ++t)
                idx[t] = *reinterpret_cast<const uint32_t*>(my_m + M_ROW * (16 * t + r) +
                                                            16 * ((wbyte >> 4) ^ m_swz_r) + (wbyte & 15)) >> msh;
            const uint4 b0 = *reinterpret_cast<const uint4*>(xr + 16 * ((8 * u + xc0) ^ r));
            const uint4 b1 = *reinterpret_cast<const uint4*>(xr + 16 * ((8 * u + xc1) ^ r));
#pragma unroll
            for (int t = 0; t < AT; ++t)
                acc[t] = Op::mma(fa[t][u], b0, b1, idx[t], acc[t]);
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

    // D[4*kg + i][l % 16] of tile t lives at red[.][t][i][kg*16 + l%16]
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
        const int ar = a0 + 16 * t + al, br = bl;
        if (ar < RA && br < RB) {
            if (sa)
                v *= sa[ar];
            if (sb)
                v *= sb[br];
            store_out<OUT>(Y, (int64_t)ar * sya + (int64_t)br * syb, v);
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
    // 17 to 64 dense rows: the tile kernels once 128-row tiles of A give
    // every CU a workgroup; until then the decode kernel, whose workgroups
    // split K and so stay many on narrow outputs
    if (RB <= 16 || (RB <= 64 && (RA + 127) / 128 < 128)) {
        const int steps = (int)(g.K / SparseOp<DT>::KSTEP);
        const int groups = (steps + kGroup - 1) / kGroup;
        // as many waves as there are load groups to split, up to 8 (measured
        // best on every decode shape: more loads in flight per CU)
        int waves = kMaxWaves;
        while (waves > 2 && groups < waves)
            waves >>= 1;
#define SP24_SKINNY(MT, XL, AT, P, NAME)                                                              \
    do {                                                                                              \
        if (!g.dry)                                                                                   \
            hipLaunchKernelGGL((sp24_skinny<DT, OUT, MT, XL, AT, P>), dim3((RA + 16 * AT - 1) / (16 * AT)), \
                               dim3(waves * 64), 0, s, av, g.a_meta, b, g.scale_a, g.scale_b, g.Y, RA, RB, \
                               g.K, sya, syb);                                                        \
        if (kname) *kname = NAME;                                                                     \
    } while (0)
        // 5 to 16 rows: the kernel that stages all 16 (4 or 8 waves; fewer
        // load groups than waves leave the extra waves idle)
#define SP24_X16(AT, NAME)                                                                            \
    do {                                                                                              \
        const dim3 grid((RA + 16 * AT - 1) / (16 * AT));                                              \
        if (!g.dry) {                                                                                 \
            if (waves <= 4)                                                                           \
                hipLaunchKernelGGL((sp24_skinny_x16<DT, OUT, AT, 4>), grid, dim3(256), 0, s, av, g.a_meta, b, \
                                   g.scale_a, g.scale_b, g.Y, RA, RB, g.K, sya, syb);                 \
            else                                                                                      \
                hipLaunchKernelGGL((sp24_skinny_x16<DT, OUT, AT, 8>), grid, dim3(512), 0, s, av, g.a_meta, b, \
                                   g.scale_a, g.scale_b, g.Y, RA, RB, g.K, sya, syb);                 \
        }                                                                                             \
        if (kname) *kname = NAME;                                                                     \
    } while (0)
        // at most 4 dense rows: stage them through LDS with contiguous 1 KiB
        // loads (a register load per step carries 64 useful bytes of 1 KiB).
        // 5 to 16: 32 rows of A per workgroup when that still leaves 192 or
        // more workgroups (each B fragment then serves two A tiles)
        const int mt = (RB + 15) / 16;
        if (RB <= 4) SP24_SKINNY(1, true, 1, 1, "sp24_skinny_x4");
        else if (mt <= 1 && tiles16 / 2 >= 192) {
            // three or more workgroups per CU: four waves each hold enough in flight
            if (tiles16 / 2 >= 3 * 256 && waves > 4)
                waves = 4;
            SP24_X16(2, "sp24_skinny_m16_a32");
        }
        else if (mt <= 1) SP24_X16(1, "sp24_skinny_m16");
        // 17 to 64: 32-row A tiles from 160 such tiles on (measured on the fp8
        // 5120-row and bf16 6144-row layers: 27-40% faster; on 4096 rows,
        // 128 tiles, 10-20% slower)
        else if (mt == 2 && tiles16 / 2 >= 160) SP24_SKINNY(2, false, 2, 1, "sp24_skinny_m32_a32");
        else if (mt == 2) SP24_SKINNY(2, false, 1, 1, "sp24_skinny_m32");
        else if (tiles16 / 2 >= 160) SP24_SKINNY(2, false, 2, 2, "sp24_skinny_m64_a32");
        else SP24_SKINNY(2, false, 1, 2, "sp24_skinny_m64");
#undef SP24_SKINNY
#undef SP24_X16
    } else {
        // the LDS-staged tile kernels, which read each B fragment once per
        // 128 or 256 rows of A
        return launch_sp24_gemm_big(g, s, kname);
    }
    return g.dry ? hipSuccess : hipGetLastError();
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
    case SP24_I8:
        if (g.out_dt == SP24_BF16) return dispatch<SP24_I8, SP24_BF16>(g, s, kname);
        return dispatch<SP24_I8, SP24_F32>(g, s, kname);
    default:
        return hipErrorInvalidValue;
    }
}

}  // namespace sp24
