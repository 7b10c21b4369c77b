// api.hip -- the extern "C" entry points of libsp24.so: argument
// validation (on the host, before any HIP call), dispatch to the kernels,
// and the sparse-versus-dense tactic selection.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "sp24_internal.h"

#define SP24_API extern "C" __attribute__((visibility("default")))

namespace sp24 {
namespace {

__global__ void fill_zero(uint8_t* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride)
        p[i] = 0;
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t s) {
    if (bytes <= 0)
        return hipSuccess;
    int64_t blocks = std::min<int64_t>((bytes + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_zero, dim3((uint32_t)blocks), dim3(256), 0, s, (uint8_t*)p, bytes);
    return hipGetLastError();
}

// Enum arguments come from C callers as ints, and C allows any int value
// there; C++ does not allow reading a value outside the enumeration's range
// as that enumeration.  Every entry point therefore reads an enum argument's
// bytes as an int and checks it before it uses the argument as the enum (the
// helpers it forwards to take the arguments by reference, so forwarding
// reads nothing).
template <class E>
int enum_bits(const E& e) {
    static_assert(sizeof(E) == sizeof(int), "the enums are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}
bool dtype_known(int v) { return v >= SP24_F16 && v <= SP24_I8; }
bool operand_known(int v) { return v == SP24_SPARSE_W || v == SP24_SPARSE_X; }

bool is_input_dtype(int dt) { return dt == SP24_F16 || dt == SP24_BF16 || dt == SP24_E4M3 || dt == SP24_I8; }

bool out_ok(sp24_dtype in, sp24_dtype out) {
    if (in == SP24_E4M3 || in == SP24_I8)
        return out == SP24_BF16 || out == SP24_F32;
    return out == SP24_F16 || out == SP24_BF16 || out == SP24_F32;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared checks of the two GEMM entry points.  Returns SP24_OK when the
// shape is eligible for the MFMA kernels.
// Checks on dtypes and sizes alone (no pointer is looked at).
sp24_status check_shape(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K, bool sparse) {
    if (!is_input_dtype(in_dt) || !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0)
        return SP24_E_SHAPE;
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2)
        return SP24_E_SHAPE;
    // the kernels address each operand with 32-bit buffer offsets, and mark
    // masked loads by adding 2^31 to an offset that may run up to one tile
    // (256 rows) past the operand: operand + 256 rows must stay below 2 GiB
    const int64_t eb = elem_bytes(in_dt), lim = (int64_t)1 << 31;
    if ((M + 256) * K * eb >= lim || (N + 256) * K * eb >= lim)
        return SP24_E_SHAPE;
    if (M == 0 || N == 0)
        return SP24_OK;
    // sparse: whole MFMA steps; dense: whole 16-byte chunks of every row
    if (K % (sparse ? gemm_k_tile(in_dt) : 16 / elem_bytes(in_dt)) != 0)
        return SP24_E_ALIGN;
    return SP24_OK;
}

sp24_status check_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K,
                       std::initializer_list<const void*> required, const void* Y,
                       const float* sx, const float* sw, bool sparse) {
    if (!is_input_dtype(in_dt) || !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0)
        return SP24_E_SHAPE;
    if (M > 0 && N > 0) {
        if (!Y)
            return SP24_E_NULL;
        if (K > 0)
            for (const void* p : required)
                if (!p)
                    return SP24_E_NULL;
    }
    sp24_status st = check_shape(in_dt, out_dt, M, N, K, sparse);
    if (st != SP24_OK || M == 0 || N == 0)
        return st;
    if (!aligned16(Y) || ((uintptr_t)sx & 3u) || ((uintptr_t)sw & 3u))
        return SP24_E_ALIGN;
    for (const void* p : required)
        if (!aligned16(p))
            return SP24_E_ALIGN;
    return SP24_OK;
}

double median(std::vector<double> v) {
    if (v.empty())
        return 0.0;
    std::sort(v.begin(), v.end());
    size_t n = v.size();
    return n % 2 ? v[n / 2] : 0.5 * (v[n / 2 - 1] + v[n / 2]);
}

}  // namespace
}  // namespace sp24

using namespace sp24;

SP24_API const char* sp24_status_str(sp24_status s) {
    switch (s) {
    case SP24_OK: return "SP24_OK";
    case SP24_E_NULL: return "SP24_E_NULL: a required pointer is NULL";
    case SP24_E_SHAPE: return "SP24_E_SHAPE: negative size, K % 4 != 0, or leading dimension < K";
    case SP24_E_DTYPE: return "SP24_E_DTYPE: unsupported dtype or dtype combination";
    case SP24_E_ALIGN: return "SP24_E_ALIGN: pointer not 16-byte aligned or K not a multiple of the GEMM K tile";
    case SP24_E_HIP: return "SP24_E_HIP: the HIP runtime reported an error";
    }
    return "unknown sp24_status";
}

SP24_API const char* sp24_version(void) { return "sp24 0.1.0 gfx950"; }

SP24_API int64_t sp24_meta_words_per_row(int64_t K) { return K < 0 ? 0 : meta_words(K); }

SP24_API sp24_status sp24_prune_compress(sp24_dtype dt, int64_t rows, int64_t K, const void* src,
                                         int64_t ld_src, void* values, uint32_t* meta,
                                         hipStream_t stream) {
    if (!dtype_known(enum_bits(dt)) || !is_input_dtype(dt))
        return SP24_E_DTYPE;
    if (rows < 0 || K < 0 || K % 4 != 0 || ld_src < K)
        return SP24_E_SHAPE;
    if (rows == 0 || K == 0)
        return SP24_OK;
    if (!src || !values || !meta)
        return SP24_E_NULL;
    return launch_prune_compress(dt, rows, K, src, ld_src, values, meta, stream) == hipSuccess
               ? SP24_OK : SP24_E_HIP;
}

SP24_API sp24_status sp24_decompress(sp24_dtype dt, int64_t rows, int64_t K, const void* values,
                                     const uint32_t* meta, void* dst, int64_t ld_dst,
                                     hipStream_t stream) {
    if (!dtype_known(enum_bits(dt)) || !is_input_dtype(dt))
        return SP24_E_DTYPE;
    if (rows < 0 || K < 0 || K % 4 != 0 || ld_dst < K)
        return SP24_E_SHAPE;
    if (rows == 0 || K == 0)
        return SP24_OK;
    if (!values || !meta || !dst)
        return SP24_E_NULL;
    return launch_decompress(dt, rows, K, values, meta, dst, ld_dst, stream) == hipSuccess
               ? SP24_OK : SP24_E_HIP;
}

// one 256-lane workgroup per row: the grid stays below 2^32 lanes
static constexpr int64_t kMaxQuantRows = (int64_t)1 << 24;

static sp24_status quantize_impl(const sp24_dtype& dt, sp24_dtype out_dt, int64_t rows, int64_t K,
                                 const void* src, int64_t ld_src, void* out, uint32_t* meta, float* scales,
                                 bool prune, hipStream_t stream) {
    if (!dtype_known(enum_bits(dt)) || (dt != SP24_F16 && dt != SP24_BF16))
        return SP24_E_DTYPE;
    if (rows < 0 || K < 0 || ld_src < K || rows > kMaxQuantRows)
        return SP24_E_SHAPE;
    if (rows == 0 || K == 0)
        return SP24_OK;
    if (!src || !out || !scales || (prune && !meta))
        return SP24_E_NULL;
    if (K % 32 != 0 || ld_src % 8 != 0 || !aligned16(src) || !aligned16(out) || (prune && !aligned16(meta)) ||
        ((uintptr_t)scales & 3u))
        return SP24_E_ALIGN;
    return launch_quantize(dt, out_dt, rows, K, src, ld_src, out, prune ? meta : nullptr, scales, stream) ==
                   hipSuccess
               ? SP24_OK : SP24_E_HIP;
}

SP24_API sp24_status sp24_quantize_prune_compress(sp24_dtype src_dt, int64_t rows, int64_t K, const void* src,
                                                  int64_t ld_src, void* values, uint32_t* meta, float* scales,
                                                  hipStream_t stream) {
    return quantize_impl(src_dt, SP24_E4M3, rows, K, src, ld_src, values, meta, scales, true, stream);
}

SP24_API sp24_status sp24_quantize_e4m3(sp24_dtype src_dt, int64_t rows, int64_t K, const void* src,
                                        int64_t ld_src, void* dst, float* scales, hipStream_t stream) {
    return quantize_impl(src_dt, SP24_E4M3, rows, K, src, ld_src, dst, nullptr, scales, false, stream);
}

SP24_API sp24_status sp24_quantize_i8_prune_compress(sp24_dtype src_dt, int64_t rows, int64_t K, const void* src,
                                                     int64_t ld_src, void* values, uint32_t* meta, float* scales,
                                                     hipStream_t stream) {
    return quantize_impl(src_dt, SP24_I8, rows, K, src, ld_src, values, meta, scales, true, stream);
}

SP24_API sp24_status sp24_quantize_i8(sp24_dtype src_dt, int64_t rows, int64_t K, const void* src,
                                      int64_t ld_src, void* dst, float* scales, hipStream_t stream) {
    return quantize_impl(src_dt, SP24_I8, rows, K, src, ld_src, dst, nullptr, scales, false, stream);
}

static sp24_status gemm_impl(const sp24_operand& which, const sp24_dtype& in_dt, const sp24_dtype& out_dt, int64_t M,
                             int64_t N, int64_t K, const void* values, const uint32_t* meta,
                             const void* dense, const float* scale_x, const float* scale_w, void* Y,
                             hipStream_t stream, const char** kname) {
    if (!operand_known(enum_bits(which)))
        return SP24_E_SHAPE;
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)))
        return SP24_E_DTYPE;
    sp24_status st = check_gemm(in_dt, out_dt, M, N, K, {values, meta, dense}, Y, scale_x, scale_w, true);
    if (st != SP24_OK)
        return st;
    if (M == 0 || N == 0)
        return SP24_OK;
    if (K == 0) {
        if (kname) *kname = "fill_zero";
        return launch_fill_zero(Y, M * N * elem_bytes(out_dt), stream) == hipSuccess ? SP24_OK : SP24_E_HIP;
    }
    GemmArgs g;
    g.in_dt = in_dt;
    g.out_dt = out_dt;
    g.M = M;
    g.N = N;
    g.K = K;
    g.a_vals = values;
    g.a_meta = meta;
    g.b = dense;
    g.a_is_w = which == SP24_SPARSE_W;
    g.scale_a = g.a_is_w ? scale_w : scale_x;
    g.scale_b = g.a_is_w ? scale_x : scale_w;
    g.Y = Y;
    return launch_sp24_gemm(g, stream, kname) == hipSuccess ? SP24_OK : SP24_E_HIP;
}

static sp24_status dense_impl(const sp24_dtype& in_dt, const sp24_dtype& out_dt, int64_t M, int64_t N, int64_t K,
                              const void* X, const void* W, const float* scale_x, const float* scale_w,
                              void* Y, hipStream_t stream, const char** kname) {
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)))
        return SP24_E_DTYPE;
    sp24_status st = check_gemm(in_dt, out_dt, M, N, K, {X, W}, Y, scale_x, scale_w, false);
    if (st != SP24_OK)
        return st;
    if (M == 0 || N == 0)
        return SP24_OK;
    if (K == 0) {
        if (kname) *kname = "fill_zero";
        return launch_fill_zero(Y, M * N * elem_bytes(out_dt), stream) == hipSuccess ? SP24_OK : SP24_E_HIP;
    }
    DenseArgs g;
    g.in_dt = in_dt;
    g.out_dt = out_dt;
    g.M = M;
    g.N = N;
    g.K = K;
    g.X = X;
    g.W = W;
    g.scale_x = scale_x;
    g.scale_w = scale_w;
    g.Y = Y;
    return launch_dense_gemm(g, stream, kname) == hipSuccess ? SP24_OK : SP24_E_HIP;
}

// Dtype and size checks of the hybrid GEMM (no pointer is looked at).
static sp24_status check_hybrid_shape(const sp24_dtype& in_dt, const sp24_dtype& out_dt, int64_t M, int64_t NS, int64_t ND,
                                      int64_t K) {
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)) || !is_input_dtype(in_dt) ||
        !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (NS < 0 || ND < 0 || NS > INT32_MAX / 2 - ND)
        return SP24_E_SHAPE;
    // both regions are at most N = NS + ND rows: the plain GEMM's limits cover them
    sp24_status st = check_shape(in_dt, out_dt, M, NS + ND, K, true);
    if (st != SP24_OK)
        return st;
    if (M > 0 && NS + ND > 0 && NS % 8 != 0)
        return SP24_E_ALIGN;
    return SP24_OK;
}

SP24_API sp24_status sp24_hybrid_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N_s, int64_t N_d,
                                      int64_t K, const void* values, const uint32_t* meta, const void* W_d,
                                      const void* X, const float* scale_x, const float* scale_w, void* Y,
                                      hipStream_t stream) {
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)) || !is_input_dtype(in_dt) ||
        !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (M < 0 || N_s < 0 || N_d < 0 || K < 0 || K % 4 != 0)
        return SP24_E_SHAPE;
    const int64_t N = N_s + N_d;
    if (M > 0 && N > 0) {
        if (!Y)
            return SP24_E_NULL;
        if (K > 0 && (!X || (N_s > 0 && (!values || !meta)) || (N_d > 0 && !W_d)))
            return SP24_E_NULL;
    }
    sp24_status st = check_hybrid_shape(in_dt, out_dt, M, N_s, N_d, K);
    if (st != SP24_OK || M == 0 || N == 0)
        return st;
    if (!aligned16(Y) || ((uintptr_t)scale_x & 3u) || ((uintptr_t)scale_w & 3u) || !aligned16(X) ||
        (N_s > 0 && (!aligned16(values) || !aligned16(meta))) || (N_d > 0 && !aligned16(W_d)))
        return SP24_E_ALIGN;
    if (K == 0)
        return launch_fill_zero(Y, M * N * elem_bytes(out_dt), stream) == hipSuccess ? SP24_OK : SP24_E_HIP;
    HybridArgs h;
    h.in_dt = in_dt;
    h.out_dt = out_dt;
    h.M = M;
    h.NS = N_s;
    h.ND = N_d;
    h.K = K;
    h.ws_vals = values;
    h.ws_meta = meta;
    h.wd = W_d;
    h.x = X;
    h.scale_x = scale_x;
    h.scale_w = scale_w;
    h.Y = Y;
    return launch_sp24_hybrid(h, stream, nullptr) == hipSuccess ? SP24_OK : SP24_E_HIP;
}

SP24_API const char* sp24_hybrid_kernel(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N_s, int64_t N_d,
                                       int64_t K) {
    if (M < 0 || K < 0 || K % 4 != 0 || check_hybrid_shape(in_dt, out_dt, M, N_s, N_d, K) != SP24_OK)
        return nullptr;
    if (M == 0 || N_s + N_d == 0)
        return "none";
    if (K == 0)
        return "fill_zero";
    HybridArgs h{};
    h.in_dt = in_dt;
    h.out_dt = out_dt;
    h.M = M;
    h.NS = N_s;
    h.ND = N_d;
    h.K = K;
    h.dry = true;
    const char* name = nullptr;
    launch_sp24_hybrid(h, nullptr, &name);
    return name;
}

// Dtype and size checks of the K-split hybrid GEMM (no pointer is looked at).
static sp24_status check_ksplit_shape(const sp24_dtype& in_dt, const sp24_dtype& out_dt, int64_t M, int64_t N,
                                      int64_t K_s, int64_t K) {
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)) || !is_input_dtype(in_dt) ||
        !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (K_s < 0 || K_s > K)
        return SP24_E_SHAPE;
    // the whole weight is N x K: the plain GEMM's limits and K tile cover both ranges
    sp24_status st = check_shape(in_dt, out_dt, M, N, K, true);
    if (st != SP24_OK)
        return st;
    // the compressed range in whole metadata blocks (8 words of a row)
    if (M > 0 && N > 0 && K_s % 256 != 0)
        return SP24_E_ALIGN;
    return SP24_OK;
}

SP24_API sp24_status sp24_ksplit_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K_s,
                                      int64_t K, const void* values, const uint32_t* meta, const void* W_d,
                                      const void* X, const float* scale_x, const float* scale_w, void* Y,
                                      hipStream_t stream) {
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)) || !is_input_dtype(in_dt) ||
        !out_ok(in_dt, out_dt))
        return SP24_E_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0 || K_s < 0 || K_s > K)
        return SP24_E_SHAPE;
    if (M > 0 && N > 0) {
        if (!Y)
            return SP24_E_NULL;
        if (K > 0 && (!X || (K_s > 0 && (!values || !meta)) || (K_s < K && !W_d)))
            return SP24_E_NULL;
    }
    sp24_status st = check_ksplit_shape(in_dt, out_dt, M, N, K_s, K);
    if (st != SP24_OK || M == 0 || N == 0)
        return st;
    if (!aligned16(Y) || ((uintptr_t)scale_x & 3u) || ((uintptr_t)scale_w & 3u) || !aligned16(X) ||
        (K_s > 0 && (!aligned16(values) || !aligned16(meta))) || (K_s < K && !aligned16(W_d)))
        return SP24_E_ALIGN;
    if (K == 0)
        return launch_fill_zero(Y, M * N * elem_bytes(out_dt), stream) == hipSuccess ? SP24_OK : SP24_E_HIP;
    KsplitArgs k;
    k.in_dt = in_dt;
    k.out_dt = out_dt;
    k.M = M;
    k.N = N;
    k.KS = K_s;
    k.K = K;
    k.ws_vals = values;
    k.ws_meta = meta;
    k.wd = W_d;
    k.x = X;
    k.scale_x = scale_x;
    k.scale_w = scale_w;
    k.Y = Y;
    return launch_sp24_ksplit(k, stream, nullptr) == hipSuccess ? SP24_OK : SP24_E_HIP;
}

SP24_API const char* sp24_ksplit_kernel(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K_s,
                                       int64_t K) {
    if (M < 0 || N < 0 || K < 0 || K % 4 != 0 || check_ksplit_shape(in_dt, out_dt, M, N, K_s, K) != SP24_OK)
        return nullptr;
    if (M == 0 || N == 0)
        return "none";
    if (K == 0)
        return "fill_zero";
    KsplitArgs k{};
    k.in_dt = in_dt;
    k.out_dt = out_dt;
    k.M = M;
    k.N = N;
    k.KS = K_s;
    k.K = K;
    k.dry = true;
    const char* name = nullptr;
    launch_sp24_ksplit(k, nullptr, &name);
    return name;
}

SP24_API const char* sp24_gemm_kernel(int sparse, sp24_operand which, sp24_dtype in_dt, sp24_dtype out_dt,
                                     int64_t M, int64_t N, int64_t K) {
    const int w = enum_bits(which);
    if (sparse && !operand_known(w))
        return nullptr;
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)))
        return nullptr;
    if (check_shape(in_dt, out_dt, M, N, K, sparse != 0) != SP24_OK)
        return nullptr;
    if (M == 0 || N == 0)
        return "none";
    if (K == 0)
        return "fill_zero";
    const char* name = nullptr;
    if (sparse) {
        GemmArgs g{};
        g.in_dt = in_dt;
        g.out_dt = out_dt;
        g.M = M;
        g.N = N;
        g.K = K;
        g.a_is_w = w == SP24_SPARSE_W;
        g.dry = true;
        launch_sp24_gemm(g, nullptr, &name);
    } else {
        DenseArgs g{};
        g.in_dt = in_dt;
        g.out_dt = out_dt;
        g.M = M;
        g.N = N;
        g.K = K;
        g.dry = true;
        launch_dense_gemm(g, nullptr, &name);
    }
    return name;
}

SP24_API sp24_status sp24_gemm(sp24_operand which, sp24_dtype in_dt, sp24_dtype out_dt, int64_t M,
                               int64_t N, int64_t K, const void* values, const uint32_t* meta,
                               const void* dense, const float* scale_x, const float* scale_w, void* Y,
                               hipStream_t stream) {
    return gemm_impl(which, in_dt, out_dt, M, N, K, values, meta, dense, scale_x, scale_w, Y, stream, nullptr);
}

SP24_API sp24_status dense_gemm(sp24_dtype in_dt, sp24_dtype out_dt, int64_t M, int64_t N, int64_t K,
                                const void* X, const void* W, const float* scale_x,
                                const float* scale_w, void* Y, hipStream_t stream) {
    return dense_impl(in_dt, out_dt, M, N, K, X, W, scale_x, scale_w, Y, stream, nullptr);
}

SP24_API sp24_status sp24_tactic_decide(int eligible, const double* t_sparse, int ns, const double* t_dense,
                                        int nd, sp24_tactic* out) {
    if (!out)
        return SP24_E_NULL;
    if (nd < 1 || !t_dense || (eligible && (ns < 1 || !t_sparse)))
        return SP24_E_SHAPE;
    out->eligible = eligible ? 1 : 0;
    out->t_dense_us = median(std::vector<double>(t_dense, t_dense + nd));
    if (!eligible) {
        out->selected = 0;
        out->t_sparse_us = 0.0;
        out->ratio = 0.0;
        if (out->reason[0] == '\0')
            snprintf(out->reason, sizeof(out->reason), "Not eligible");
        return SP24_OK;
    }
    out->t_sparse_us = median(std::vector<double>(t_sparse, t_sparse + ns));
    const double ts = out->t_sparse_us;
    out->ratio = ts > 0.0 ? out->t_dense_us / ts : 0.0;
    // latency is the sole criterion: sparse only if strictly faster
    out->selected = ts < out->t_dense_us ? 1 : 0;
    if (out->selected)
        snprintf(out->reason, sizeof(out->reason), "Sparse kernel %.2fx faster", out->ratio);
    else if (ts == out->t_dense_us)
        snprintf(out->reason, sizeof(out->reason), "Tie: dense kept (sparse not faster)");
    else
        snprintf(out->reason, sizeof(out->reason), "Dense kernel %.2fx faster", ts / out->t_dense_us);
    return SP24_OK;
}

SP24_API sp24_status sp24_audit_aggregate(const sp24_tactic* records, const int64_t* layer_counts,
                                          int64_t n_records, double other_time_us, sp24_audit_metrics* out) {
    if (!out)
        return SP24_E_NULL;
    if (n_records < 0 || !std::isfinite(other_time_us) || other_time_us < 0.0)
        return SP24_E_SHAPE;
    if (n_records > 0 && (!records || !layer_counts))
        return SP24_E_NULL;
    sp24_audit_metrics m{};
    double total = 0.0;
    for (int64_t i = 0; i < n_records; ++i) {
        const sp24_tactic& r = records[i];
        const int64_t c = layer_counts[i];
        const double ts = r.t_sparse_us + r.t_compress_us;
        if (c < 0 || !std::isfinite(ts) || !std::isfinite(r.t_dense_us) || r.t_sparse_us < 0.0 ||
            r.t_compress_us < 0.0 || r.t_dense_us < 0.0)
            return SP24_E_SHAPE;
        m.candidate_layers += c;
        if (r.eligible)
            m.eligible_layers += c;
        if (r.eligible && r.selected) {
            m.sparse_selected_layers += c;
            m.sparse_gpu_time_us += (double)c * ts;
            total += (double)c * ts;
        } else {
            total += (double)c * r.t_dense_us;
        }
    }
    m.dense_fallback_layers = m.candidate_layers - m.sparse_selected_layers;
    m.total_gpu_time_us = total + other_time_us;
    m.eligibility_ratio = m.candidate_layers ? (double)m.eligible_layers / (double)m.candidate_layers : 0.0;
    m.sparse_selection_ratio =
        m.eligible_layers ? (double)m.sparse_selected_layers / (double)m.eligible_layers : 0.0;
    m.sparse_gpu_time_coverage = m.total_gpu_time_us > 0.0 ? m.sparse_gpu_time_us / m.total_gpu_time_us : 0.0;
    *out = m;
    return SP24_OK;
}

SP24_API sp24_status sp24_select_tactic(sp24_operand which, sp24_dtype in_dt, sp24_dtype out_dt, int64_t M,
                                        int64_t N, int64_t K, const void* values, const uint32_t* meta,
                                        const void* dense_other, const void* dense_pruned,
                                        const float* scale_x, const float* scale_w, void* Y_scratch,
                                        int warmup, int reps, hipStream_t stream, sp24_tactic* out) {
    if (!out)
        return SP24_E_NULL;
    memset(out, 0, sizeof(*out));
    if (reps < 1 || warmup < 0)
        return SP24_E_SHAPE;
    if (!operand_known(enum_bits(which)))
        return SP24_E_SHAPE;
    if (!dtype_known(enum_bits(in_dt)) || !dtype_known(enum_bits(out_dt)))
        return SP24_E_DTYPE;
    // eligibility of the sparse path
    int eligible = 1;
    if (!is_input_dtype(in_dt) || !out_ok(in_dt, out_dt)) {
        eligible = 0;
        snprintf(out->reason, sizeof(out->reason), "Unsupported dtype");
    } else {
        sp24_status st = check_gemm(in_dt, out_dt, M, N, K, {values, meta, dense_other}, Y_scratch,
                                    scale_x, scale_w, true);
        if (st == SP24_E_ALIGN) {
            eligible = 0;
            snprintf(out->reason, sizeof(out->reason), "Alignment failure");
        } else if (st != SP24_OK) {
            return st;
        }
    }
    const void* X = which == SP24_SPARSE_W ? dense_other : dense_pruned;
    const void* W = which == SP24_SPARSE_W ? dense_pruned : dense_other;
    sp24_status dst = check_gemm(in_dt, out_dt, M, N, K, {X, W}, Y_scratch, scale_x, scale_w, false);
    if (dst != SP24_OK)
        return dst;   // the dense path must run: nothing to fall back to otherwise

    const char* sname = nullptr;
    const char* dname = nullptr;
    auto run_sparse = [&](hipEvent_t mid) -> sp24_status {
        if (which == SP24_SPARSE_X) {
            sp24_status st = sp24_prune_compress(in_dt, M, K, dense_pruned, K, const_cast<void*>(values),
                                                 const_cast<uint32_t*>(meta), stream);
            if (st != SP24_OK)
                return st;
        }
        if (mid && hipEventRecord(mid, stream) != hipSuccess)
            return SP24_E_HIP;
        return gemm_impl(which, in_dt, out_dt, M, N, K, values, meta, dense_other, scale_x, scale_w,
                         Y_scratch, stream, &sname);
    };
    auto run_dense = [&]() -> sp24_status {
        return dense_impl(in_dt, out_dt, M, N, K, X, W, scale_x, scale_w, Y_scratch, stream, &dname);
    };

    // per rep: sparse start, split (after compress), end; dense start, split, end.  The dense
    // side records a split too, right at its start, so that both measurements hold the same
    // number of event markers: a marker between two events is itself timed, and on small
    // kernels one extra marker on one side only would bias the choice.
    constexpr size_t kEv = 6;
    std::vector<hipEvent_t> ev((size_t)reps * kEv, nullptr);
    sp24_status result = SP24_OK;
    for (auto& e : ev)
        if (hipEventCreate(&e) != hipSuccess) {
            result = SP24_E_HIP;
            break;
        }
    std::vector<double> ts, tc, tg, td;
    if (result == SP24_OK) {
        for (int i = 0; i < warmup && result == SP24_OK; ++i) {
            if (eligible)
                result = run_sparse(nullptr);
            if (result == SP24_OK)
                result = run_dense();
        }
        // interleave the two paths rep by rep so that clock and thermal drift hit both
        for (int i = 0; i < reps && result == SP24_OK; ++i) {
            hipEvent_t* e = &ev[(size_t)i * kEv];
            if (eligible) {
                if (hipEventRecord(e[0], stream) != hipSuccess) { result = SP24_E_HIP; break; }
                result = run_sparse(e[1]);
                if (result != SP24_OK) break;
                if (hipEventRecord(e[2], stream) != hipSuccess) { result = SP24_E_HIP; break; }
            }
            if (hipEventRecord(e[3], stream) != hipSuccess || hipEventRecord(e[5], stream) != hipSuccess) {
                result = SP24_E_HIP;
                break;
            }
            result = run_dense();
            if (result != SP24_OK) break;
            if (hipEventRecord(e[4], stream) != hipSuccess) { result = SP24_E_HIP; break; }
        }
        if (result == SP24_OK && hipStreamSynchronize(stream) != hipSuccess)
            result = SP24_E_HIP;
        for (int i = 0; i < reps && result == SP24_OK; ++i) {
            hipEvent_t* e = &ev[(size_t)i * kEv];
            float a = 0.f, b = 0.f, c = 0.f;
            if (eligible) {
                if (hipEventElapsedTime(&a, e[0], e[1]) != hipSuccess ||
                    hipEventElapsedTime(&b, e[1], e[2]) != hipSuccess) {
                    result = SP24_E_HIP;
                    break;
                }
                tc.push_back(1e3 * a);
                tg.push_back(1e3 * b);
                ts.push_back(1e3 * (a + b));
            }
            if (hipEventElapsedTime(&c, e[3], e[4]) != hipSuccess) {
                result = SP24_E_HIP;
                break;
            }
            td.push_back(1e3 * c);
        }
    }
    for (auto& e : ev)
        if (e)
            (void)hipEventDestroy(e);
    if (result != SP24_OK)
        return result;
    char reason[96];
    memcpy(reason, out->reason, sizeof(reason));
    result = sp24_tactic_decide(eligible, ts.data(), (int)ts.size(), td.data(), (int)td.size(), out);
    if (result != SP24_OK)
        return result;
    if (!eligible)
        memcpy(out->reason, reason, sizeof(reason));
    if (eligible && which == SP24_SPARSE_X) {
        out->t_compress_us = median(tc);
        out->t_sparse_us = median(tg);
    }
    const char* chosen = out->selected ? sname : dname;
    snprintf(out->kernel, sizeof(out->kernel), "%s", chosen ? chosen : "none");
    return SP24_OK;
}
