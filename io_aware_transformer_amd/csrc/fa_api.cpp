// C ABI of the attention library: argument validation, kernel dispatch and
// error reporting.  Every check runs on the host before any HIP call, so an
// invalid call launches nothing and touches no device state.
#include "fa.h"
#include "fa_internal.h"

#include <climits>
#include <cmath>
#include <cstdint>

namespace {

thread_local int g_last_hip_error = 0;

int hip_failure(hipError_t e) {
    g_last_hip_error = int(e);
    return FA_ERR_HIP;
}

constexpr float kLog2e = 1.4426950408889634f;

// The kernels work with scale * log2(e): a finite scale whose product
// overflows (|scale| above about 2.36e38) is rejected with the non-finite ones.
bool scale_ok(float scale) { return std::isfinite(scale) && std::isfinite(scale * kLog2e); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape / scalar checks shared by fa_fwd and fa_bwd.
int validate(int B, int Hq, int Hkv, int N, int d, float scale, int causal, int dtype) {
    if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_DTYPE;
    if (B < 0 || N < 0 || N > FA_MAX_N) return FA_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq > FA_MAX_HEADS || Hkv > Hq || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (!scale_ok(scale)) return FA_ERR_ARG;
    // Grid bound: query blocks of 32 rows at the finest, times batch x heads.
    const long long blocks = fa::sat_mul(fa::sat_mul(((long long)N + 31) / 32, B), Hq);
    if (blocks > (long long)INT_MAX) return FA_ERR_SHAPE;
    return FA_OK;
}

// Checks of the split forward: N_q queries against N_k keys.
int validate_split(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int dtype, int splits) {
    if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_DTYPE;
    if (B < 0 || Nq < 0 || Nk < 0 || Nq > FA_MAX_N || Nk > FA_MAX_N) return FA_ERR_SHAPE;
    if (Hq < 1 || Hkv < 1 || Hq > FA_MAX_HEADS || Hkv > Hq || Hq % Hkv != 0) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    if (!scale_ok(scale)) return FA_ERR_ARG;
    if (splits < 0 || splits > FA_MAX_SPLITS) return FA_ERR_ARG;
    if (B > 0 && Nq > 0 && Nk == 0) return FA_ERR_SHAPE;  // attention over no keys is undefined
    return FA_OK;
}

// Resolved number of key ranges (0 = the default for these sizes), or 0 when
// there is nothing to do.
int split_parts(int B, int Hq, int Hkv, int Nq, int Nk, int d, int splits) {
    if (B == 0 || Nq == 0) return 0;
    return splits > 0 ? splits : fa::split_parts_default(B, Hq, Hkv, Nq, Nk, d);
}

// Window bounds -> kernel form.  -1: unbounded; -2: no mask at all (the
// unmasked kernels).  A bound of N - 1 or more hides nothing on its side
// (|i - j| <= N - 1 for rows of one sequence), so it is the unbounded case:
// this keeps the kernels' index arithmetic (row +- bound) far from int
// overflow for any int bound.  Returns whether the masked kernels are needed.
bool window_bounds(int left, int right, int N, int& wl, int& wr) {
    if (left == -2 && right == -2) {
        wl = wr = fa::kUnbounded;
        return false;
    }
    const bool lu = left < 0 || left >= N - 1, ru = right < 0 || right >= N - 1;
    wl = lu ? fa::kUnbounded : left;
    wr = ru ? fa::kUnbounded : right;
    return !(lu && ru);  // unbounded on both sides is no mask
}

// Fixed-length batches pass cu == nullptr; packed sequences pass the device
// offsets, the packed row count `total` and the longest length as N.
// Dropout of the dropout entry points (t8 = 0: none).
struct Drop {
    int t8 = 0;
    unsigned long long seed = 0;
    unsigned int offset = 0;
};

int fwd_impl(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int N, int d,
             float scale, int left, int right, int dtype, void* stream, const int* cu = nullptr, int total = 0,
             const unsigned char* bmask = nullptr, Drop drop = Drop()) {
    if (B == 0 || N == 0) return FA_OK;
    if (!Q || !K || !V || !O) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 16))
        return FA_ERR_ALIGN;
    fa::FwdParams p{};
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.O = O;
    p.LSE = LSE;
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.cu = cu;
    p.total = total;
    p.scale_log2 = scale * kLog2e;
    bool masked = window_bounds(left, right, N, p.wl, p.wr);
    if (bmask != nullptr) {
        p.bmask = bmask;
        p.nb = (N + fa::kSparseBlock - 1) / fa::kSparseBlock;
        masked = true;
    }
    p.drop_t8 = drop.t8;
    p.drop_k0 = uint32_t(drop.seed & 0xFFFFFFFFull);
    p.drop_k1 = uint32_t(drop.seed >> 32);
    p.drop_off = drop.offset;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = (dtype == FA_BF16) ? fa::launch_fwd_bf16(p, d, masked, s) : fa::launch_fwd_f32(p, d, masked, s);
    if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
    if (e != hipSuccess) return hip_failure(e);
    return FA_OK;
}

int bwd_impl(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
             void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv, int N, int d,
             float scale, int left, int right, int dtype, void* stream, const int* cu = nullptr, int total = 0,
             const unsigned char* bmask = nullptr, Drop drop = Drop(), bool allow_split = true) {
    if (dtype == FA_BF16 && d == 256) return FA_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return FA_OK;
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
        !aligned(LSE, 16) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16))
        return FA_ERR_ALIGN;
    const long long rows = cu != nullptr ? (long long)total : (long long)B * N;
    // Grouped heads of a fixed-length batch: the query heads of a key/value
    // head may be split over more dK/dV workgroups, whose float partials
    // live in the workspace after the D term.
    const int hsplit = (cu == nullptr && allow_split && dtype == FA_BF16) ? fa::bwd_hsplit(B, H_q, H_kv, N) : 1;
    const size_t need = hsplit > 1 ? fa::bwd_workspace_bytes_split(B, H_q, H_kv, N, d)
                                   : fa::bwd_workspace_bytes(H_q, rows);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
    fa::BwdParams p{};
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.O = O;
    p.dO = dO;
    p.LSE = LSE;
    p.dQ = dQ;
    p.dK = dK;
    p.dV = dV;
    p.Drow = static_cast<float*>(workspace);
    p.hsplit = hsplit;
    if (hsplit > 1) {
        const size_t dbytes = fa::bwd_workspace_bytes(H_q, rows);
        const size_t kv_elems = size_t(B) * H_kv * N * d;
        const size_t part = (size_t(hsplit) * kv_elems * sizeof(float) + 255) / 256 * 256;
        p.dk_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + dbytes);
        p.dv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + dbytes + part);
        p.part_stride = kv_elems;
    }
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.N = N;
    p.cu = cu;
    p.total = total;
    p.scale = scale;
    p.scale_log2 = scale * kLog2e;
    bool masked = window_bounds(left, right, N, p.wl, p.wr);
    if (bmask != nullptr) {
        p.bmask = bmask;
        p.nb = (N + fa::kSparseBlock - 1) / fa::kSparseBlock;
        masked = true;
    }
    p.drop_t8 = drop.t8;
    p.drop_k0 = uint32_t(drop.seed & 0xFFFFFFFFull);
    p.drop_k1 = uint32_t(drop.seed >> 32);
    p.drop_off = drop.offset;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = (dtype == FA_BF16) ? fa::launch_bwd_bf16(p, d, masked, s) : fa::launch_bwd_f32(p, d, masked, s);
    if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
    if (e != hipSuccess) return hip_failure(e);
    return FA_OK;
}

// Checks of the packed (variable-length) entry points beyond validate():
// the packed row count and the offsets array.  Returns FA_OK or an error;
// `work` tells whether there is anything to compute.
int validate_varlen(const int* cu, int batch, int total, int max_seqlen, bool& work) {
    if (total < 0) return FA_ERR_SHAPE;
    work = batch > 0 && total > 0 && max_seqlen > 0;
    if (!work) return FA_OK;
    if (!cu) return FA_ERR_NULL;
    if (!aligned(cu, 4)) return FA_ERR_ALIGN;
    return FA_OK;
}

bool split_grid_ok(int B, int Hq, int Hkv, int Nq, int parts) {
    const long long rows = (long long)(Hq / Hkv) * Nq;
    const long long blocks = fa::sat_mul(fa::sat_mul(fa::sat_mul(B, Hkv), (rows + 31) / 32), parts);  // one wave each
    const long long merge_rows = fa::sat_mul(fa::sat_mul(B, Hq), Nq);
    return blocks <= (long long)INT_MAX && merge_rows <= (long long)INT_MAX * 4;
}

}  // namespace

namespace fa {

hipError_t set_max_dynamic_lds(const void* kern, size_t bytes, DeviceOnce& once) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t(1) << dev) : 0;
    if (bit != 0 && (once.done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
    if (e == hipSuccess && bit != 0) once.done.fetch_or(bit, std::memory_order_release);
    return e;
}

int device_cu_count() {
    constexpr int kDefault = 256;
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();  // clear the sticky error of a host without devices
        return kDefault;
    }
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = kDefault;
    }
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace fa

extern "C" {

int fa_version(void) { return 130; }

const char* fa_status_str(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_NULL: return "FA_ERR_NULL";
        case FA_ERR_SHAPE: return "FA_ERR_SHAPE";
        case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM";
        case FA_ERR_DTYPE: return "FA_ERR_DTYPE";
        case FA_ERR_ALIGN: return "FA_ERR_ALIGN";
        case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
        case FA_ERR_HIP: return "FA_ERR_HIP";
        case FA_ERR_ARG: return "FA_ERR_ARG";
        default: return "FA_ERR_UNKNOWN";
    }
}

int fa_last_hip_error(void) { return g_last_hip_error; }

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int N, int d,
           float scale, int causal, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    return fwd_impl(Q, K, V, O, LSE, B, H_q, H_kv, N, d, scale, causal ? -1 : -2, causal ? 0 : -2, dtype, stream);
}

int fa_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int N,
                  int d, float scale, int window_left, int window_right, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, 0, dtype);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
    return fwd_impl(Q, K, V, O, LSE, B, H_q, H_kv, N, d, scale, window_left, window_right, dtype, stream);
}

size_t fa_bwd_workspace_size(int B, int H_q, int H_kv, int N, int d, int dtype) {
    if (validate(B, H_q, H_kv, N, d, 1.0f, 0, dtype) != FA_OK) return 0;
    if (B == 0 || N == 0) return 0;
    return dtype == FA_BF16 ? fa::bwd_workspace_bytes_split(B, H_q, H_kv, N, d)
                            : fa::bwd_workspace_bytes(H_q, (long long)B * N);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
           void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv, int N, int d,
           float scale, int causal, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H_q, H_kv, N, d, scale,
                    causal ? -1 : -2, causal ? 0 : -2, dtype, stream);
}

int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                   void* dQ, void* dK, void* dV, int B, int H_q, int H_kv, int N, int d, float scale, int causal,
                   int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_BF16 && d == 256) return FA_ERR_UNSUPPORTED;
    if (B == 0 || N == 0) return FA_OK;
    static_assert(fa::kNoAllocScratchBytes == size_t(FA_NOALLOC_MAX_ROWS) * sizeof(float), "limit and buffer agree");
    if ((long long)B * H_q * N > (long long)FA_NOALLOC_MAX_ROWS) return FA_ERR_WORKSPACE;
    if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULL;
    hipError_t e = hipSuccess;
    void* scratch = fa::noalloc_scratch(e);
    if (scratch == nullptr) return hip_failure(e);
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, scratch, fa::kNoAllocScratchBytes, B, H_q, H_kv, N, d, scale,
                    causal ? -1 : -2, causal ? 0 : -2, dtype, stream, nullptr, 0, nullptr, Drop(), false);
}

int fa_bwd_window(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                  void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv,
                  int N, int d, float scale, int window_left, int window_right, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, 0, dtype);
    if (st != FA_OK) return st;
    if (window_left < -1 || window_right < -1) return FA_ERR_ARG;
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H_q, H_kv, N, d, scale,
                    window_left, window_right, dtype, stream);
}

// Checks of the block-sparse entry points beyond validate().
static int validate_sparse(const unsigned char* bmask, int B, int N, int d, int dtype, bool& work) {
    if (dtype != FA_BF16 || (d != 64 && d != 128) || N > FA_SPARSE_MAX_N) return FA_ERR_UNSUPPORTED;
    work = B > 0 && N > 0;
    if (work && !bmask) return FA_ERR_NULL;
    return FA_OK;
}

int fa_fwd_blocksparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                       const unsigned char* block_mask, int B, int H_q, int H_kv, int N, int d, float scale,
                       int causal, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    bool work = false;
    if ((st = validate_sparse(block_mask, B, N, d, dtype, work)) != FA_OK || !work) return st;
    return fwd_impl(Q, K, V, O, LSE, B, H_q, H_kv, N, d, scale, -1, causal ? 0 : -1, dtype, stream, nullptr, 0,
                    block_mask);
}

int fa_bwd_blocksparse(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                       void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes,
                       const unsigned char* block_mask, int B, int H_q, int H_kv, int N, int d, float scale,
                       int causal, int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    bool work = false;
    if ((st = validate_sparse(block_mask, B, N, d, dtype, work)) != FA_OK || !work) return st;
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H_q, H_kv, N, d, scale, -1,
                    causal ? 0 : -1, dtype, stream, nullptr, 0, block_mask);
}

// Dropout probability -> 8-bit threshold t8 = round(p * 256) (half to
// even); FA_ERR_ARG unless 0 <= t8 <= 255.
static int dropout_t8(float p, int& t8) {
    if (!std::isfinite(p) || p < 0.f) return FA_ERR_ARG;
    const double x = std::nearbyint(double(p) * 256.0);
    if (x > 255.0) return FA_ERR_ARG;
    t8 = int(x);
    return FA_OK;
}

int fa_fwd_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int N,
                   int d, float scale, int causal, float dropout_p, unsigned long long seed, unsigned int offset,
                   int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    Drop dr;
    if ((st = dropout_t8(dropout_p, dr.t8)) != FA_OK) return st;
    if (dtype != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    dr.seed = seed;
    dr.offset = offset;
    return fwd_impl(Q, K, V, O, LSE, B, H_q, H_kv, N, d, scale, causal ? -1 : -2, causal ? 0 : -2, dtype, stream,
                    nullptr, 0, nullptr, dr);
}

int fa_bwd_dropout(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                   void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, int B, int H_q, int H_kv,
                   int N, int d, float scale, int causal, float dropout_p, unsigned long long seed, unsigned int offset,
                   int dtype, void* stream) {
    int st = validate(B, H_q, H_kv, N, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    Drop dr;
    if ((st = dropout_t8(dropout_p, dr.t8)) != FA_OK) return st;
    if (dtype != FA_BF16 || (d != 64 && d != 128)) return FA_ERR_UNSUPPORTED;
    dr.seed = seed;
    dr.offset = offset;
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H_q, H_kv, N, d, scale,
                    causal ? -1 : -2, causal ? 0 : -2, dtype, stream, nullptr, 0, nullptr, dr);
}

int fa_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE, const int* cu_seqlens, int batch,
                  int total, int max_seqlen, int H_q, int H_kv, int d, float scale, int causal, int dtype,
                  void* stream) {
    int st = validate(batch, H_q, H_kv, max_seqlen, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    bool work = false;
    if ((st = validate_varlen(cu_seqlens, batch, total, max_seqlen, work)) != FA_OK || !work) return st;
    return fwd_impl(Q, K, V, O, LSE, batch, H_q, H_kv, max_seqlen, d, scale, causal ? -1 : -2, causal ? 0 : -2, dtype,
                    stream, cu_seqlens, total);
}

size_t fa_bwd_varlen_workspace_size(int total, int H_q, int H_kv, int d, int dtype) {
    if (validate(1, H_q, H_kv, 0, d, 1.0f, 0, dtype) != FA_OK || total <= 0) return 0;
    return fa::bwd_workspace_bytes(H_q, total);
}

int fa_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE,
                  void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, const int* cu_seqlens,
                  int batch, int total, int max_seqlen, int H_q, int H_kv, int d, float scale, int causal, int dtype,
                  void* stream) {
    int st = validate(batch, H_q, H_kv, max_seqlen, d, scale, causal, dtype);
    if (st != FA_OK) return st;
    if (dtype == FA_BF16 && d == 256) return FA_ERR_UNSUPPORTED;
    bool work = false;
    if ((st = validate_varlen(cu_seqlens, batch, total, max_seqlen, work)) != FA_OK || !work) return st;
    return bwd_impl(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, batch, H_q, H_kv, max_seqlen, d,
                    scale, causal ? -1 : -2, causal ? 0 : -2, dtype, stream, cu_seqlens, total);
}

size_t fa_fwd_split_workspace_size(int B, int H_q, int H_kv, int N_q, int N_k, int d, int num_splits, int dtype) {
    if (validate_split(B, H_q, H_kv, N_q, N_k, d, 1.0f, 0, dtype, num_splits) != FA_OK) return 0;
    const int parts = split_parts(B, H_q, H_kv, N_q, N_k, d, num_splits);
    if (parts == 0) return 0;
    return fa::split_workspace_bytes(B, H_q, N_q, d, parts);
}

int fa_fwd_split_parts(int B, int H_q, int H_kv, int N_q, int N_k, int d, int num_splits) {
    if (validate_split(B, H_q, H_kv, N_q, N_k, d, 1.0f, 0, FA_BF16, num_splits) != FA_OK) return 0;
    return split_parts(B, H_q, H_kv, N_q, N_k, d, num_splits);
}

int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int N_q,
                 int N_k, int d, float scale, int causal, int num_splits, void* workspace, size_t workspace_bytes,
                 int dtype, void* stream) {
    int st = validate_split(B, H_q, H_kv, N_q, N_k, d, scale, causal, dtype, num_splits);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16 || d == 256) return FA_ERR_UNSUPPORTED;
    const int parts = split_parts(B, H_q, H_kv, N_q, N_k, d, num_splits);
    if (parts == 0) return FA_OK;
    if (!split_grid_ok(B, H_q, H_kv, N_q, parts)) return FA_ERR_SHAPE;
    if (!Q || !K || !V || !O) return FA_ERR_NULL;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 16))
        return FA_ERR_ALIGN;
    const size_t need = fa::split_workspace_bytes(B, H_q, N_q, d, parts);
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
    const long long rows = (long long)B * H_q * N_q;
    fa::SplitParams p{};
    p.Q = Q;
    p.K = K;
    p.V = V;
    p.Opart = static_cast<float*>(workspace);
    p.LSEpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         (size_t(parts) * size_t(rows) * d * sizeof(float) + 255) / 256 * 256);
    p.B = B;
    p.Hq = H_q;
    p.Hkv = H_kv;
    p.Nq = N_q;
    p.Nk = N_k;
    p.scale_log2 = scale * kLog2e;
    p.parts = parts;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = fa::launch_fwd_split_bf16(p, d, causal, s);
    if (e == hipSuccess) e = fa::launch_lse_merge(p.Opart, p.LSEpart, parts, rows, d, O, LSE, 1, s);
    if (e == hipErrorNotSupported) return FA_ERR_UNSUPPORTED;
    if (e != hipSuccess) return hip_failure(e);
    return FA_OK;
}

int fa_lse_merge(const float* O_parts, const float* LSE_parts, int num_parts, long long rows, int d, void* O,
                 float* LSE, int dtype, void* stream) {
    if (dtype != FA_BF16 && dtype != FA_FP32) return FA_ERR_DTYPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
    if (num_parts < 1 || num_parts > FA_MAX_SPLITS) return FA_ERR_ARG;
    if (rows < 0 || rows > (long long)INT_MAX * 4) return FA_ERR_SHAPE;
    if (rows == 0) return FA_OK;
    if (!O_parts || !LSE_parts || !O) return FA_ERR_NULL;
    if (!aligned(O_parts, 16) || !aligned(LSE_parts, 16) || !aligned(O, 16) || !aligned(LSE, 16)) return FA_ERR_ALIGN;
    hipError_t e = fa::launch_lse_merge(O_parts, LSE_parts, num_parts, rows, d, O, LSE, dtype == FA_BF16,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_failure(e);
    return FA_OK;
}

}  // extern "C"
