// sp24_internal.h -- declarations shared by the HIP kernels and the C-ABI
// glue of libsp24.so.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sp24.h"

namespace sp24 {

// ------------------------------------------------------------------ types
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) __bf16 bf16x16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) _Float16 f16x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

inline int elem_bytes(sp24_dtype dt) { return dt == SP24_E4M3 || dt == SP24_I8 ? 1 : (dt == SP24_F32 ? 4 : 2); }
inline int64_t meta_words(int64_t K) { return (K + 31) / 32; }

// K consumed by one sparse MFMA step, per input dtype: 64 for 16-bit
// (v_smfmac_*_16x16x64), 128 for fp8 (v_smfmac_*_16x16x128).
inline int64_t gemm_k_tile(sp24_dtype dt) { return elem_bytes(dt) == 1 ? 128 : 64; }

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; arguments were validated by
// the caller.
hipError_t launch_prune_compress(sp24_dtype dt, int64_t rows, int64_t K, const void* src,
                                 int64_t ld_src, void* values, uint32_t* meta, hipStream_t s);
hipError_t launch_decompress(sp24_dtype dt, int64_t rows, int64_t K, const void* values,
                             const uint32_t* meta, void* dst, int64_t ld_dst, hipStream_t s);

// Per-row quantization of a 16-bit operand to out_dt (SP24_E4M3 or SP24_I8):
// codes into `out` (rows x K, meta == nullptr) or, fused with the 2:4 prune,
// kept codes into `out` (rows x K/2) and metadata into `meta`; one fp32 scale
// per row into `scales`.
hipError_t launch_quantize(sp24_dtype dt, sp24_dtype out_dt, int64_t rows, int64_t K, const void* src,
                           int64_t ld_src, void* out, uint32_t* meta, float* scales, hipStream_t s);

struct GemmArgs {
    sp24_dtype in_dt, out_dt;
    int64_t M, N, K;
    const void* a_vals;      // compressed operand values (rows x K/2)
    const uint32_t* a_meta;  // its metadata (rows x K/32)
    const void* b;           // dense operand (cols x K)
    const float* scale_a;    // per compressed-operand row, or null
    const float* scale_b;    // per dense-operand row, or null
    void* Y;                 // M x N
    int a_is_w;              // 1: compressed operand is W (rows = N), 0: it is X (rows = M)
    bool dry = false;        // only report the kernel that would be launched
};
// Sparse GEMM; writes the name of the kernel it launched into kname (if
// non-null).  With g.dry set, launches nothing and returns hipSuccess.
hipError_t launch_sp24_gemm(const GemmArgs& g, hipStream_t s, const char** kname);
// The LDS-staged tile kernels (256 x 256 down to 128 x 64 tiles) for outputs
// with more than 16 dense rows (called by launch_sp24_gemm).
hipError_t launch_sp24_gemm_big(const GemmArgs& g, hipStream_t s, const char** kname);

// The hybrid GEMM: Y (M x (NS + ND)), columns [0, NS) = X * Ws^T with Ws
// compressed, columns [NS, NS + ND) = X * Wd^T with Wd dense; one launch.
struct HybridArgs {
    sp24_dtype in_dt, out_dt;
    int64_t M, NS, ND, K;
    const void* ws_vals;      // NS x K/2
    const uint32_t* ws_meta;  // NS x K/32
    const void* wd;           // ND x K
    const void* x;            // M x K
    const float* scale_x;     // M, or null
    const float* scale_w;     // NS + ND, or null
    void* Y;
    bool dry = false;
};
hipError_t launch_sp24_hybrid(const HybridArgs& h, hipStream_t s, const char** kname);

// The K-split hybrid GEMM: Y (M x N) = X * W^T with W's columns [0, KS)
// compressed (ws_vals N x KS/2, ws_meta N x KS/32) and [KS, K) dense (wd,
// N x (K - KS)); one launch, both ranges into the same accumulators.
struct KsplitArgs {
    sp24_dtype in_dt, out_dt;
    int64_t M, N, KS, K;
    const void* ws_vals;
    const uint32_t* ws_meta;
    const void* wd;
    const void* x;            // M x K
    const float* scale_x;     // M, or null
    const float* scale_w;     // N, or null
    void* Y;
    bool dry = false;
};
hipError_t launch_sp24_ksplit(const KsplitArgs& k, hipStream_t s, const char** kname);

struct DenseArgs {
    sp24_dtype in_dt, out_dt;
    int64_t M, N, K;
    const void* X;
    const void* W;
    const float* scale_x;
    const float* scale_w;
    void* Y;
    bool dry = false;        // only report the kernel that would be launched
};
hipError_t launch_dense_gemm(const DenseArgs& g, hipStream_t s, const char** kname);
// The LDS-staged dense tile kernels (called by launch_dense_gemm).
hipError_t launch_dense_gemm_big(const DenseArgs& g, hipStream_t s, const char** kname);

}  // namespace sp24
