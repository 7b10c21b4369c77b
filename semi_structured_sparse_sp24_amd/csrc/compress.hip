// compress.hip -- magnitude 2:4 prune + compress, and decompress, for gfx950.
//
// Prune rule ("2:4 Structured Sparsity Explained", "How to make a model 2:4
// sparse"): in every group of four consecutive elements along K keep the two
// of largest magnitude; ties go to the lower index.  Compressed form ("How
// 2:4 sparsity works"): the two kept values, half the storage, plus a 2-bit
// position for each.  The fused one-pass form (read the operand once, write
// values and positions once) follows section 3.5 of the 2:4-versus-
// quantization paper.
//
// Magnitude is compared on integer keys: the sign-stripped bit pattern (for
// the sign-magnitude float formats) or |x| (for two's complement int8, so
// -128 ranks above 127), made unique by appending (3 - position) as two low
// bits, so "larger key" means
// "larger magnitude, or equal magnitude at a lower position".  The kept pair
// is then the largest and second-largest of four distinct integers.
//
// Work unit of the fast kernels: 16 bytes of dense input (8 x 16-bit or 16 x
// 8-bit elements = 2 or 4 groups) -> 8 bytes of values + 1 or 2 bytes of
// metadata.  Lanes of a wave take consecutive units, so every load is one
// contiguous 1 KiB per wave instruction and every store is contiguous too.
// HBM traffic per dense element: 2 + 1 + 0.125 = 3.125 B (16-bit) or
// 1 + 0.5 + 0.125 = 1.625 B (fp8, int8).
#include "sp24_internal.h"

namespace sp24 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerThread = 4;

// Kept positions (p0 < p1) of one group from its four magnitude keys.
__device__ __forceinline__ void top2(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3,
                                     uint32_t& p0, uint32_t& p1) {
    uint32_t c0 = (k0 << 2) | 3u, c1 = (k1 << 2) | 2u, c2 = (k2 << 2) | 1u, c3 = (k3 << 2) | 0u;
    uint32_t hi01 = max(c0, c1), lo01 = min(c0, c1);
    uint32_t hi23 = max(c2, c3), lo23 = min(c2, c3);
    uint32_t first = max(hi01, hi23);
    uint32_t second = max(min(hi01, hi23), max(lo01, lo23));
    uint32_t pa = 3u - (first & 3u), pb = 3u - (second & 3u);
    p0 = min(pa, pb);
    p1 = max(pa, pb);
}

template <typename T>
__device__ __forceinline__ T pick(uint32_t p, T e0, T e1, T e2, T e3) {
    return p == 0 ? e0 : (p == 1 ? e1 : (p == 2 ? e2 : e3));
}

// One group of 16-bit elements (e0..e3 in the low halves): returns the packed
// pair (v0 | v1 << 16) and the nibble.
__device__ __forceinline__ uint32_t group16(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3,
                                            uint32_t& nib) {
    uint32_t p0, p1;
    top2(e0 & 0x7fffu, e1 & 0x7fffu, e2 & 0x7fffu, e3 & 0x7fffu, p0, p1);
    nib = p0 | (p1 << 2);
    return pick(p0, e0, e1, e2, e3) | (pick(p1, e0, e1, e2, e3) << 16);
}

// Magnitude key of one byte: fp8 (sign-magnitude) or int8 (two's complement).
template <bool INT8>
__device__ __forceinline__ uint32_t mag8(uint32_t e) {
    if (INT8)
        return e & 0x80u ? 256u - e : e;    // |x|, 0 .. 128
    return e & 0x7fu;
}

// One group of 8-bit elements: returns the packed pair (v0 | v1 << 8).
template <bool INT8>
__device__ __forceinline__ uint32_t group8(uint32_t e0, uint32_t e1, uint32_t e2, uint32_t e3,
                                           uint32_t& nib) {
    uint32_t p0, p1;
    top2(mag8<INT8>(e0), mag8<INT8>(e1), mag8<INT8>(e2), mag8<INT8>(e3), p0, p1);
    nib = p0 | (p1 << 2);
    return pick(p0, e0, e1, e2, e3) | (pick(p1, e0, e1, e2, e3) << 8);
}

// ---------------------------------------------------------------- fast path
// Requires K*eb % 16 == 0, 16-byte aligned src rows, 8-byte aligned values.
template <int EB, bool INT8>
__global__ void __launch_bounds__(kThreads)
prune_compress_units(const uint8_t* __restrict__ src, int64_t ld_bytes, uint32_t units_per_row,
                     uint32_t total_units, uint8_t* __restrict__ values, int64_t vrow_bytes,
                     uint8_t* __restrict__ meta, int64_t mrow_bytes, uint32_t meta_used_bytes) {
    const uint32_t base = blockIdx.x * (kThreads * kUnitsPerThread) + threadIdx.x;
    uint4 in[kUnitsPerThread];
    uint32_t row[kUnitsPerThread], col[kUnitsPerThread];
#pragma unroll
    for (int j = 0; j < kUnitsPerThread; ++j) {
        uint32_t u = base + j * kThreads;
        row[j] = u / units_per_row;
        col[j] = u - row[j] * units_per_row;
        if (u < total_units)
            in[j] = *reinterpret_cast<const uint4*>(src + row[j] * ld_bytes + (int64_t)col[j] * 16);
    }
#pragma unroll
    for (int j = 0; j < kUnitsPerThread; ++j) {
        uint32_t u = base + j * kThreads;
        if (u >= total_units)
            continue;
        uint32_t w[4] = {in[j].x, in[j].y, in[j].z, in[j].w};
        uint2 out;
        uint8_t* mrow = meta + row[j] * mrow_bytes;
        if (EB == 2) {
            uint32_t n0, n1;
            out.x = group16(w[0] & 0xffffu, w[0] >> 16, w[1] & 0xffffu, w[1] >> 16, n0);
            out.y = group16(w[2] & 0xffffu, w[2] >> 16, w[3] & 0xffffu, w[3] >> 16, n1);
            mrow[col[j]] = (uint8_t)(n0 | (n1 << 4));
        } else {
            uint32_t n[4], pr[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                pr[g] = group8<INT8>(w[g] & 0xffu, (w[g] >> 8) & 0xffu, (w[g] >> 16) & 0xffu, w[g] >> 24, n[g]);
            out.x = pr[0] | (pr[1] << 16);
            out.y = pr[2] | (pr[3] << 16);
            *reinterpret_cast<uint16_t*>(mrow + 2 * col[j]) =
                (uint16_t)(n[0] | (n[1] << 4) | (n[2] << 8) | (n[3] << 12));
        }
        *reinterpret_cast<uint2*>(values + row[j] * vrow_bytes + (int64_t)col[j] * 8) = out;
        // zero the unused tail of the row's last metadata word
        if (col[j] == units_per_row - 1)
            for (uint32_t b = meta_used_bytes; b < (uint32_t)mrow_bytes; ++b)
                mrow[b] = 0;
    }
}

template <int EB>
__global__ void __launch_bounds__(kThreads)
decompress_units(const uint8_t* __restrict__ values, int64_t vrow_bytes,
                 const uint8_t* __restrict__ meta, int64_t mrow_bytes, uint32_t units_per_row,
                 uint32_t total_units, uint8_t* __restrict__ dst, int64_t ld_bytes) {
    const uint32_t base = blockIdx.x * (kThreads * kUnitsPerThread) + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kUnitsPerThread; ++j) {
        uint32_t u = base + j * kThreads;
        if (u >= total_units)
            continue;
        uint32_t row = u / units_per_row, col = u - row * units_per_row;
        uint2 v = *reinterpret_cast<const uint2*>(values + row * vrow_bytes + (int64_t)col * 8);
        uint4 out;
        if (EB == 2) {
            uint32_t m = meta[row * mrow_bytes + col];
            uint32_t o[4];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                uint32_t pair = g ? v.y : v.x;
                uint32_t nib = (m >> (4 * g)) & 0xfu, p0 = nib & 3u, p1 = nib >> 2;
                uint32_t a = pair & 0xffffu, b = pair >> 16;
                uint32_t e[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    e[i] = (i == (int)p1) ? b : ((i == (int)p0) ? a : 0u);
                o[2 * g] = e[0] | (e[1] << 16);
                o[2 * g + 1] = e[2] | (e[3] << 16);
            }
            out = make_uint4(o[0], o[1], o[2], o[3]);
        } else {
            uint32_t m = *reinterpret_cast<const uint16_t*>(meta + row * mrow_bytes + 2 * col);
            uint32_t o[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                uint32_t pair = ((g < 2 ? v.x : v.y) >> (16 * (g & 1))) & 0xffffu;
                uint32_t nib = (m >> (4 * g)) & 0xfu, p0 = nib & 3u, p1 = nib >> 2;
                uint32_t a = pair & 0xffu, b = pair >> 8;
                uint32_t r = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    r |= ((i == (int)p1) ? b : ((i == (int)p0) ? a : 0u)) << (8 * i);
                o[g] = r;
            }
            out = make_uint4(o[0], o[1], o[2], o[3]);
        }
        *reinterpret_cast<uint4*>(dst + row * ld_bytes + (int64_t)col * 16) = out;
    }
}

// ---------------------------------------------------------------- general path
// Any K % 4 == 0, any strides and alignments: one thread per metadata word
// (up to 8 groups), element-wise loads and stores.
template <int EB, bool INT8>
__global__ void __launch_bounds__(kThreads)
prune_compress_words(const uint8_t* __restrict__ src, int64_t ld, int64_t rows, int64_t K,
                     uint8_t* __restrict__ values, uint32_t* __restrict__ meta) {
    const int64_t mw = (K + 31) / 32;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= rows * mw)
        return;
    const int64_t r = t / mw, w = t - r * mw;
    const int64_t groups = K / 4;
    uint32_t word = 0;
    for (int q = 0; q < 8; ++q) {
        int64_t g = w * 8 + q;
        if (g >= groups)
            break;
        uint32_t e[4];
        for (int i = 0; i < 4; ++i) {
            const uint8_t* p = src + (r * ld + 4 * g + i) * EB;
            e[i] = EB == 2 ? (uint32_t)p[0] | ((uint32_t)p[1] << 8) : (uint32_t)p[0];
        }
        uint32_t nib, pr;
        pr = EB == 2 ? group16(e[0], e[1], e[2], e[3], nib) : group8<INT8>(e[0], e[1], e[2], e[3], nib);
        uint8_t* v = values + (r * (K / 2) + 2 * g) * EB;
        for (int b = 0; b < 2 * EB; ++b)
            v[b] = (uint8_t)(pr >> (8 * b));
        word |= nib << (4 * q);
    }
    meta[r * mw + w] = word;
}

template <int EB>
__global__ void __launch_bounds__(kThreads)
decompress_words(const uint8_t* __restrict__ values, const uint32_t* __restrict__ meta,
                 int64_t rows, int64_t K, uint8_t* __restrict__ dst, int64_t ld) {
    const int64_t mw = (K + 31) / 32;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= rows * mw)
        return;
    const int64_t r = t / mw, w = t - r * mw;
    const int64_t groups = K / 4;
    const uint32_t word = meta[r * mw + w];
    for (int q = 0; q < 8; ++q) {
        int64_t g = w * 8 + q;
        if (g >= groups)
            break;
        uint32_t nib = (word >> (4 * q)) & 0xfu, p0 = nib & 3u, p1 = nib >> 2;
        const uint8_t* v = values + (r * (K / 2) + 2 * g) * EB;
        uint8_t* d = dst + (r * ld + 4 * g) * EB;
        for (int i = 0; i < 4; ++i) {
            const uint8_t* s = (i == (int)p1) ? v + EB : ((i == (int)p0) ? v : nullptr);
            for (int b = 0; b < EB; ++b)
                d[i * EB + b] = s ? s[b] : 0;
        }
    }
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace

hipError_t launch_prune_compress(sp24_dtype dt, int64_t rows, int64_t K, const void* src,
                                 int64_t ld_src, void* values, uint32_t* meta, hipStream_t s) {
    if (rows == 0 || K == 0)
        return hipSuccess;
    const int eb = elem_bytes(dt);
    const int64_t row_bytes = K * eb;
    const int64_t units = rows * (row_bytes / 16);
    const bool fast = row_bytes % 16 == 0 && (ld_src * eb) % 16 == 0 && aligned(src, 16) &&
                      aligned(values, 8) && aligned(meta, 4) && units < (int64_t)UINT32_MAX - 4096;
    if (fast) {
        uint32_t upr = (uint32_t)(row_bytes / 16);
        uint32_t blocks = (uint32_t)((units + kThreads * kUnitsPerThread - 1) / (kThreads * kUnitsPerThread));
        auto kern = eb == 2 ? prune_compress_units<2, false>
                            : (dt == SP24_I8 ? prune_compress_units<1, true> : prune_compress_units<1, false>);
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const uint8_t*)src, ld_src * eb,
                           upr, (uint32_t)units, (uint8_t*)values, row_bytes / 2, (uint8_t*)meta,
                           meta_words(K) * 4, (uint32_t)(K / 8));
    } else {
        int64_t threads = rows * meta_words(K);
        uint32_t blocks = (uint32_t)((threads + kThreads - 1) / kThreads);
        auto kern = eb == 2 ? prune_compress_words<2, false>
                            : (dt == SP24_I8 ? prune_compress_words<1, true> : prune_compress_words<1, false>);
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const uint8_t*)src, ld_src, rows,
                           K, (uint8_t*)values, meta);
    }
    return hipGetLastError();
}

hipError_t launch_decompress(sp24_dtype dt, int64_t rows, int64_t K, const void* values,
                             const uint32_t* meta, void* dst, int64_t ld_dst, hipStream_t s) {
    if (rows == 0 || K == 0)
        return hipSuccess;
    const int eb = elem_bytes(dt);
    const int64_t row_bytes = K * eb;
    const int64_t units = rows * (row_bytes / 16);
    const bool fast = row_bytes % 16 == 0 && (ld_dst * eb) % 16 == 0 && aligned(dst, 16) &&
                      aligned(values, 8) && aligned(meta, 4) && units < (int64_t)UINT32_MAX - 4096;
    if (fast) {
        uint32_t upr = (uint32_t)(row_bytes / 16);
        uint32_t blocks = (uint32_t)((units + kThreads * kUnitsPerThread - 1) / (kThreads * kUnitsPerThread));
        auto kern = eb == 2 ? decompress_units<2> : decompress_units<1>;
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const uint8_t*)values, row_bytes / 2,
                           (const uint8_t*)meta, meta_words(K) * 4, upr, (uint32_t)units,
                           (uint8_t*)dst, ld_dst * eb);
    } else {
        int64_t threads = rows * meta_words(K);
        uint32_t blocks = (uint32_t)((threads + kThreads - 1) / kThreads);
        auto kern = eb == 2 ? decompress_words<2> : decompress_words<1>;
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), 0, s, (const uint8_t*)values, meta, rows,
                           K, (uint8_t*)dst, ld_dst);
    }
    return hipGetLastError();
}

}  // namespace sp24
