// quantize.hip -- per-row quantization of a 16-bit operand to fp8 (e4m3) or
// int8, fused with the magnitude 2:4 prune and compress for dynamic
// activations.
//
// The online path of the 2:4-versus-quantization paper (section 3.5, "Measuring
// speed", and 4.2, "Speed", which lists 2:4 with FP8 and with INT8): the
// activation is quantized, pruned and compressed in one pass that reads it
// once and writes the kept values and their indices once; one scale per row
// (section 2, "Quantization").  Per row, with Q = 448 (e4m3) or 127 (int8):
//   s = max|x| / Q     (1 for an all-zero row; a NaN does not count), in fp32;
//   q = code(x / s)    x / s in fp32 (correctly rounded division), then
//                      e4m3: round to nearest even to OCP e4m3fn, saturating
//                            at 448;
//                      int8: round to the nearest integer, ties to even,
//                            saturated to [-127, 127]; a NaN codes to 0;
//   prune: in every group of four codes keep the two of largest magnitude
//   (ties to the lower index) -- the codes are what the GEMM consumes, so the
//   selection is made on them.
// The plain variant writes all codes (the dense GEMM's input).
//
// A workgroup of 256 lanes per row.  Lane t takes the 16-element chunks
// t, t + 256, ... (two 16-byte loads each) and keeps them in registers: the
// row is read from memory once, its maximum found with a wave reduction and
// four LDS words, and the codes formed from the registers.  Rows longer than
// 256 * kMaxChunks chunks are taken in rounds and read twice.
//
// Codes without the division.  With y = 1/s (correctly rounded, once per row,
// then lowered by 2^-21 relative) t = x * y lies below x / s in magnitude, by
// 5 to 11 units of 2^-24 relative; so the fp32 quotient q lies strictly above
// t and at most 23 fp32 ulps of t beyond it, and |t| < Q.
//   e4m3: rounding is monotone, so when t and the fp32 value 32 ulps beyond
//   it (its bit pattern + 32) convert to the same code, so does every value
//   between them, q included, and the hardware conversion of t is the code.
//   int8: |q - t| < 2^-13 (|q| <= 128), so when t lies more than 2^-12 from
//   the nearest half-integer, q rounds to the same integer as t.
// Otherwise the four elements of that word take the correctly rounded
// quotient (Markstein's fused-multiply-add correction, below), which the same
// conversions code exactly (it lies at most an ulp beyond Q).  Such near-ties are not rare: a 16-bit x over a 16-bit maximum
// often lands exactly on an e4m3 midpoint (about one element in 200 of a
// Gaussian bf16 row in e4m3, one in 2500 in int8).  Rows holding an infinity
// or a NaN, or whose scale is below the fp32 normals, take the division and a
// bitwise encoder for every element.
#include "sp24_internal.h"

namespace sp24 {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;     // four waves per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxChunks = 8;     // 16-element chunks a lane holds at once

__device__ __forceinline__ float bits_to_float(uint32_t h, sp24_dtype dt) {
    if (dt == SP24_BF16)
        return __builtin_bit_cast(float, h << 16);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> e4m3fn code by its bit pattern: round to nearest even, saturating
// at 448 (0x7e); NaN -> 0x7f.  The exact path for the few values the
// conversion instruction is not trusted with.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7fffffffu;
    if (mag > 0x7f800000u)
        return 0x7fu;
    if (mag >= 0x43e00000u)                     // |v| >= 448
        return sign | 0x7eu;
    const int e = (int)(mag >> 23) - 127;
    uint32_t code;
    if (e < -6) {
        // below the smallest normal: a multiple of 2^-9, rounded to even
        const float t = __builtin_bit_cast(float, mag) * 512.0f;   // exact scaling
        code = (uint32_t)__builtin_rintf(t);                        // 0 .. 8 (8 = smallest normal)
    } else {
        const uint32_t man = mag & 0x7fffffu;
        uint32_t keep = man >> 20;
        const uint32_t rest = man & 0xfffffu;
        keep += (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
        code = ((uint32_t)(e + 7) << 3) + keep;                     // a carry moves to the exponent
    }
    return sign | code;
}

// The e4m3 codes of four fp32 values, element order from the low byte.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    // the low-half conversion keeps the old high half, which the second one replaces
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float above(float t) {   // 32 ulps further from zero
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, t) + 32u);
}

__device__ __forceinline__ uint32_t pmax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pmin(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// The 2:4 selection on two groups of four codes at once (group A in the low
// 16-bit half, group B in the high half).  Key of position i: code magnitude
// in the high byte, 3 - i in the low byte, so the larger key is the larger
// magnitude and, among equals, the lower index.  Returns the kept positions
// p0 < p1 of each group, one per half (p0 in `lo`, p1 in `hi`).
__device__ __forceinline__ void top2_pair(uint32_t A, uint32_t B, uint32_t& lo, uint32_t& hi) {
    uint32_t k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // bytes: 0, A.byte i, 0, B.byte i   (selector 12 gives a zero byte)
        const uint32_t p = __builtin_amdgcn_perm(B, A, 0x000c000cu | ((uint32_t)i << 8) | ((uint32_t)(4 + i) << 24));
        k[i] = (p & 0x7f007f00u) | ((uint32_t)(3 - i) * 0x00010001u);
    }
    const uint32_t hi01 = pmax(k[0], k[1]), lo01 = pmin(k[0], k[1]);
    const uint32_t hi23 = pmax(k[2], k[3]), lo23 = pmin(k[2], k[3]);
    const uint32_t first = pmax(hi01, hi23);
    const uint32_t second = pmax(pmin(hi01, hi23), pmax(lo01, lo23));
    const uint32_t pa = (first & 0x00030003u) ^ 0x00030003u;     // 3 - (3 - i)
    const uint32_t pb = (second & 0x00030003u) ^ 0x00030003u;
    lo = pmin(pa, pb);
    hi = pmax(pa, pb);
}

// The two code formats.  fast4: the codes of four values t = x * y (element
// order from the low byte) and whether any of them must be redone exactly;
// convert4: the codes of four quotients of a finite row (within an ulp of
// the code range, where the fast conversion is exact); exact: the code of any
// fp32 quotient (non-finite and saturating ones included); mag: per byte, the
// magnitude the 2:4 selection ranks (top2_pair reads its low seven bits).
template <sp24_dtype OUT>
struct Codec;

template <>
struct Codec<SP24_E4M3> {
    static constexpr float kQ = 448.0f;
    static __device__ __forceinline__ uint32_t fast4(const float (&t)[4], bool& redo) {
        const uint32_t q = cvt4(t[0], t[1], t[2], t[3]);
        redo = q != cvt4(above(t[0]), above(t[1]), above(t[2]), above(t[3]));
        return q;
    }
    // a finite row's quotient can exceed 448 by an ulp (s rounded down), where the clamp gives the
    // code that rounding with saturation gives
    static __device__ __forceinline__ uint32_t convert4(const float (&q)[4]) {
        float c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            c[j] = __builtin_fminf(__builtin_fmaxf(q[j], -448.0f), 448.0f);
        return cvt4(c[0], c[1], c[2], c[3]);
    }
    static __device__ __forceinline__ uint32_t exact(float v) { return e4m3_rne_sat(v); }
    static __device__ __forceinline__ uint32_t mag(uint32_t w) { return w; }   // sign-magnitude bytes
};

template <>
struct Codec<SP24_I8> {
    static constexpr float kQ = 127.0f;
    // adding 1.5 * 2^23 rounds to an integer, ties to even, and leaves it
    // (two's complement, |v| < 2^22) in the low mantissa bits
    static __device__ __forceinline__ uint32_t pack4(const uint32_t (&b)[4]) {
        return __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                     __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
    }
    static __device__ __forceinline__ uint32_t fast4(const float (&t)[4], bool& redo) {
        uint32_t b[4];
        bool r = false;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float m = t[j] + 0x1.8p23f;
            r = r || __builtin_fabsf(t[j] - (m - 0x1.8p23f)) > 0.5f - 0x1p-12f;
            b[j] = __builtin_bit_cast(uint32_t, m);
        }
        redo = r;
        return pack4(b);
    }
    static __device__ __forceinline__ uint32_t convert4(const float (&q)[4]) {
        uint32_t b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = __builtin_bit_cast(uint32_t, q[j] + 0x1.8p23f);
        return pack4(b);
    }
    static __device__ __forceinline__ uint32_t exact(float v) {
        if (__builtin_isnan(v))
            return 0u;
        const float r = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
        return (uint32_t)(int)r & 0xffu;
    }
    // |q| per byte: codes are never -128, so (q ^ 0xff) + 1 stays within the byte
    static __device__ __forceinline__ uint32_t mag(uint32_t w) {
        const uint32_t sg = (w >> 7) & 0x01010101u;
        return (w ^ (sg * 0xffu)) + sg;
    }
};

// Maximum over the 64 lanes, in every lane: a prefix maximum within each row
// of 16 lanes (DPP row shifts, the lanes shifted in from outside the row read
// 0), the row results carried across rows by the row broadcasts, then lane 63.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));   // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));   // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));   // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));   // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));   // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));   // row_bcast:31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Maximum over the workgroup (one row); every lane gets it.  `red` holds one
// word per wave and must not be the words the previous reduction read.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v, uint32_t* red) {
    v = wave_max_u32(v);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    return max(max(red[0], red[1]), max(red[2], red[3]));
}

// One row per workgroup, CH chunks per lane and round.  PRUNE: write kept
// codes + metadata; else write every code.
template <sp24_dtype DT, sp24_dtype OUT, bool PRUNE, int CH>
__global__ void __launch_bounds__(kThreads)
quantize_rows(const uint8_t* __restrict__ src, int64_t ld_bytes, int64_t K,
              uint8_t* __restrict__ out, uint8_t* __restrict__ meta, float* __restrict__ scales) {
    __shared__ uint32_t red[2][kWaves];       // [maximum, NaN-free maximum][wave]
    const int lr = threadIdx.x;
    const int64_t chunks = K / 16;
    constexpr int64_t kRound = (int64_t)kThreads * CH;
    // fewer than kMaxChunks per lane: the launch chose CH so that one round covers the row
    const int rounds = CH < kMaxChunks ? 1 : (int)((chunks + kRound - 1) / kRound);
    constexpr uint32_t kInf = DT == SP24_BF16 ? 0x7f80u : 0x7c00u;   // magnitude bits of +inf

    auto load = [&](uint4 (&a)[CH], uint4 (&b)[CH], int64_t row, int rd) {
        const uint8_t* r = src + row * ld_bytes;
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int64_t c = rd * kRound + u * kThreads + lr;
            const bool in = c < chunks;
            a[u] = in ? *reinterpret_cast<const uint4*>(r + 32 * c) : make_uint4(0, 0, 0, 0);
            b[u] = in ? *reinterpret_cast<const uint4*>(r + 32 * c + 16) : make_uint4(0, 0, 0, 0);
        }
    };

    uint4 a[CH], b[CH];
    const int64_t row = blockIdx.x;
    {
        const uint8_t* r = src + row * ld_bytes;
        // ---- max |x| as magnitude bits (ordered like the values), two halves per word
        uint32_t mx = 0;
        for (int rd = 0; rd < rounds; ++rd) {
            load(a, b, row, rd);
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const uint32_t w[8] = {a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    mx = pmax(mx, w[i] & 0x7fff7fffu);
            }
        }
        const uint32_t amax_raw = row_max_u32(max(mx & 0xffffu, mx >> 16), red[0]);
        uint32_t amax = amax_raw;
        if (amax_raw > kInf) {
            // a NaN is in the row: the maximum is taken over the other elements
            uint32_t m = 0;
            for (int64_t c = lr; c < chunks; c += kThreads) {
                const uint4 p = *reinterpret_cast<const uint4*>(r + 32 * c);
                const uint4 q = *reinterpret_cast<const uint4*>(r + 32 * c + 16);
                const uint32_t w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t l = w[i] & 0x7fffu, h = (w[i] >> 16) & 0x7fffu;
                    m = max(m, l <= kInf ? l : 0u);
                    m = max(m, h <= kInf ? h : 0u);
                }
            }
            amax = row_max_u32(m, red[1]);
        }
        const float s = amax ? __fdiv_rn(bits_to_float(amax, DT), Codec<OUT>::kQ) : 1.0f;
        const float y0 = __fdiv_rn(1.0f, s);
        const float y = y0 * (1.0f - 0x1p-21f);
        const bool exact_row = amax_raw >= kInf || !(s >= 0x1p-126f);
        if (lr == 0)
            scales[row] = s;

        // ---- codes, selection, stores
        for (int rd = 0; rd < rounds; ++rd) {
            if (rounds > 1)
                load(a, b, row, rd);
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int64_t c = rd * kRound + u * kThreads + lr;
                if (c >= chunks)
                    continue;
                const uint32_t w[8] = {a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w};
                float x[16];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    x[2 * i] = bits_to_float(w[i] & 0xffffu, DT);
                    x[2 * i + 1] = bits_to_float(w[i] >> 16, DT);
                }
                uint32_t qw[4];                 // four codes per word, element order
                bool any = false;
                bool redo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        t[j] = x[4 * i + j] * y;
                    qw[i] = Codec<OUT>::fast4(t, redo[i]);
                    any = any || redo[i];
                }
                if (exact_row) {
                    // non-finite or tiny-scale rows: every code from the division and the bitwise encoder
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t q = 0;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            q |= Codec<OUT>::exact(__fdiv_rn(x[4 * i + j], s)) << (8 * j);
                        qw[i] = q;
                    }
                } else if (any) {
                    // a finite row: the correctly rounded quotients lie within the code range, where the
                    // fast conversion is exact.  The quotient by Markstein's correction of x * RN(1/s):
                    // q0 = RN(x y0), r = x - q0 s (exact, one fma), q = RN(q0 + r y0), with x's sign
                    // (which fixes -0 / s).  Exact where no intermediate falls below the fp32 normals,
                    // and checked on the GPU against the division, code for code, for every bf16 and
                    // f16 element and maximum whose scale is an fp32 normal; a word holding an element
                    // below 2^-100 in magnitude (other than 0) takes the division instead.
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (redo[i]) {
                            bool tiny = false;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                tiny = tiny || (x[4 * i + j] != 0.0f && __builtin_fabsf(x[4 * i + j]) < 0x1p-100f);
                            float q[4];
                            if (tiny) {
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    q[j] = __fdiv_rn(x[4 * i + j], s);
                            } else {
#pragma unroll
                                for (int j = 0; j < 4; ++j) {
                                    const float v = x[4 * i + j];
                                    const float q0 = __fmul_rn(v, y0);
                                    const float r = __builtin_fmaf(-q0, s, v);
                                    const float qm = __builtin_fmaf(r, y0, q0);
                                    q[j] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, qm) & 0x7fffffffu) |
                                                                        (__builtin_bit_cast(uint32_t, v) & 0x80000000u));
                                }
                            }
                            qw[i] = Codec<OUT>::convert4(q);
                        }
                    }
                }
                if (PRUNE) {
                    uint32_t vw[2], nib = 0;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint32_t p0, p1;
                        top2_pair(Codec<OUT>::mag(qw[2 * h]), Codec<OUT>::mag(qw[2 * h + 1]), p0, p1);
                        const uint32_t n = p0 | (p1 << 2);           // a metadata nibble per half
                        nib |= ((n & 0xfu) | ((n >> 12) & 0xf0u)) << (8 * h);
                        // bytes p of qw[2h] are selector values 0..3, of qw[2h+1] 4..7
                        vw[h] = __builtin_amdgcn_perm(qw[2 * h + 1], qw[2 * h], p0 | (p1 << 8) | 0x04040000u);
                    }
                    *reinterpret_cast<uint2*>(out + row * (K / 2) + 8 * c) = make_uint2(vw[0], vw[1]);
                    // 16 elements = half a metadata word: lanes 2i and 2i+1 fill word i
                    *reinterpret_cast<uint16_t*>(meta + row * (K / 8) + 2 * c) = (uint16_t)nib;
                } else {
                    *reinterpret_cast<uint4*>(out + row * K + 16 * c) = make_uint4(qw[0], qw[1], qw[2], qw[3]);
                }
            }
        }
    }
}

template <sp24_dtype DT, sp24_dtype OUT, bool PRUNE, int CH>
void launch_shape(int64_t rows, int64_t K, const uint8_t* src, int64_t ld_bytes, uint8_t* out, uint8_t* meta,
                  float* scales, hipStream_t s) {
    hipLaunchKernelGGL((quantize_rows<DT, OUT, PRUNE, CH>), dim3((uint32_t)rows), dim3(kThreads), 0, s, src,
                       ld_bytes, K, out, meta, scales);
}

// Chunks per lane: the whole row in registers up to K = 32768, longer rows in rounds.
template <sp24_dtype DT, sp24_dtype OUT, bool PRUNE>
hipError_t launch_dt(int64_t rows, int64_t K, const uint8_t* src, int64_t ld_bytes, uint8_t* out, uint8_t* meta,
                     float* scales, hipStream_t s) {
    const int64_t chunks = K / 16;
    if (chunks <= kThreads)
        launch_shape<DT, OUT, PRUNE, 1>(rows, K, src, ld_bytes, out, meta, scales, s);
    else if (chunks <= 2 * kThreads)
        launch_shape<DT, OUT, PRUNE, 2>(rows, K, src, ld_bytes, out, meta, scales, s);
    else if (chunks <= 4 * kThreads)
        launch_shape<DT, OUT, PRUNE, 4>(rows, K, src, ld_bytes, out, meta, scales, s);
    else
        launch_shape<DT, OUT, PRUNE, kMaxChunks>(rows, K, src, ld_bytes, out, meta, scales, s);
    return hipGetLastError();
}

template <sp24_dtype OUT, bool PRUNE>
hipError_t launch(sp24_dtype dt, int64_t rows, int64_t K, const void* src, int64_t ld_src, void* out,
                  uint32_t* meta, float* scales, hipStream_t s) {
    const int64_t ld_bytes = ld_src * 2;
    if (dt == SP24_BF16)
        return launch_dt<SP24_BF16, OUT, PRUNE>(rows, K, (const uint8_t*)src, ld_bytes, (uint8_t*)out,
                                                (uint8_t*)meta, scales, s);
    return launch_dt<SP24_F16, OUT, PRUNE>(rows, K, (const uint8_t*)src, ld_bytes, (uint8_t*)out, (uint8_t*)meta,
                                           scales, s);
}

}  // namespace

hipError_t launch_quantize(sp24_dtype dt, sp24_dtype out_dt, int64_t rows, int64_t K, const void* src,
                           int64_t ld_src, void* out, uint32_t* meta, float* scales, hipStream_t s) {
    if (out_dt == SP24_I8)
        return meta ? launch<SP24_I8, true>(dt, rows, K, src, ld_src, out, meta, scales, s)
                    : launch<SP24_I8, false>(dt, rows, K, src, ld_src, out, nullptr, scales, s);
    return meta ? launch<SP24_E4M3, true>(dt, rows, K, src, ld_src, out, meta, scales, s)
                : launch<SP24_E4M3, false>(dt, rows, K, src, ld_src, out, nullptr, scales, s);
}

}  // namespace sp24
