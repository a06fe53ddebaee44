// Host-side interface between the C ABI (fa_api.cpp) and the kernel
// launchers.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace fa {

// Forward launch parameters.  Pointers are device pointers; element type is
// bf16 or float depending on the launcher.  scale_log2 = scale * log2(e).
struct FwdParams {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    float* LSE;  // may be null
    int B, Hq, Hkv, N;
    float scale_log2;
    int nqb;    // number of query blocks (filled by the launcher)
    int qmode;  // bf16 kernel: 0 use Q, 1 negate Q, 2 zero Q (filled by the launcher)
    // Window of the masked kernels: query i sees key j when
    // i - wl <= j <= i + wr (kUnbounded on a side without a bound).  The
    // causal mask is (kUnbounded, 0).  Unused by the unmasked kernels.
    int wl, wr;
    // Packed sequences: when cu is non-null, Q/O are [Hq, total, d], K/V
    // [Hkv, total, d], LSE [Hq, total], and sequence b is rows cu[b] ..
    // cu[b+1]-1 of every head (cu is a device array of B + 1 ints); N is then
    // the longest sequence (the grid's row bound).
    const int* cu;
    int total;
    // Block-sparse map (MASK 3 kernels): nb x nb bytes in device memory,
    // nb = ceil(N / kSparseBlock); query i sees key j only when
    // bmask[(i / kSparseBlock) * nb + j / kSparseBlock] != 0 (and the window
    // (wl, wr) allows it).
    const unsigned char* bmask;
    int nb;
    // Dropout on P (drop_t8 > 0): element kept when its Philox byte >= drop_t8;
    // key (drop_k0, drop_k1), counter word 3 drop_off.
    int drop_t8;
    uint32_t drop_k0, drop_k1, drop_off;
};

constexpr int kUnbounded = 1 << 30;
// Block-sparse attention: positions per map block, and the longest sequence
// the kernels' per-workgroup tile lists (64-row / 64-key tiles, in LDS) hold.
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxN = 1 << 16;
constexpr int kSparseListCap = kSparseMaxN / 64;

// Backward launch parameters.
struct BwdParams {
    const void* Q;
    const void* K;
    const void* V;
    const void* O;
    const void* dO;
    const float* LSE;
    void* dQ;
    void* dK;
    void* dV;
    float* Drow;  // workspace: D_i = dO_i . O_i, float [B, Hq, N]
    int B, Hq, Hkv, N;
    float scale;       // softmax scale
    float scale_log2;  // scale * log2(e)
    int nqb, nkb;      // query / key blocks (filled by the launchers)
    int wl, wr;        // window of the masked kernels, as FwdParams
    const int* cu;     // packed sequences, as FwdParams (Drow is then [Hq, total])
    int total;
    const unsigned char* bmask;  // block-sparse map, as FwdParams
    int nb;
    int drop_t8;  // dropout, as FwdParams
    uint32_t drop_k0, drop_k1, drop_off;
    // Grouped heads: the dK/dV kernels split each key/value head's group of
    // query heads into hsplit slices (workgroups of their own) that write
    // float partials (dk_part / dv_part + slice * part_stride, indexed like
    // dK / dV), summed in slice order by a reduction kernel.  1: no split,
    // results straight to dK / dV.
    int hsplit;
    float* dk_part;
    float* dv_part;
    size_t part_stride;
};

// Split key/value forward parameters.  Q [B, Hq, Nq, d], K/V [B, Hkv, Nk, d]
// (bf16); the partials go to Opart fp32 [parts][B*Hq*Nq][d] and LSEpart fp32
// [parts][B*Hq*Nq].
struct SplitParams {
    const void* Q;
    const void* K;
    const void* V;
    float* Opart;
    float* LSEpart;
    int B, Hq, Hkv, Nq, Nk;
    float scale_log2;
    int parts;  // key ranges
    int qmode;  // filled by the launcher (as FwdParams::qmode)
    int chunk;  // keys per range, a multiple of 32 (filled by the launcher)
    int nrb;    // blocks of 32 packed rows per kv head (filled by the launcher)
};

// Each launcher enqueues its kernels on `stream` and returns the first HIP
// error (hipSuccess when everything was enqueued).  Shapes were validated
// by the caller; d is one of the supported head dims for that launcher.
// `causal` selects the masked kernels, which apply the window (wl, wr).
hipError_t launch_fwd_bf16(FwdParams p, int d, int causal, hipStream_t stream);
hipError_t launch_fwd_f32(FwdParams p, int d, int causal, hipStream_t stream);
hipError_t launch_bwd_bf16(BwdParams p, int d, int causal, hipStream_t stream);
hipError_t launch_bwd_f32(BwdParams p, int d, int causal, hipStream_t stream);

// Workspace bytes of the backward for `rows` query rows per head, summed
// over the batch (B * N for a fixed-length batch, total for packed
// sequences): the D term only.
size_t bwd_workspace_bytes(int Hq, long long rows);
// Query-head slices per key/value head of a fixed-length backward (a power
// of two dividing H_q / H_kv; 1 unless the dK/dV grid would leave compute
// units idle), and the workspace bytes including the float partials.
int bwd_hsplit(int B, int Hq, int Hkv, int N);
size_t bwd_workspace_bytes_split(int B, int Hq, int Hkv, int N, int d);

// Allocation-free backward: size of the fixed per-device buffer that holds
// the D_i term (float [B, Hq, N] rows, 256-byte aligned), and its device
// address on the current device (nullptr and `err` set on failure).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
void* noalloc_scratch(hipError_t& err);

// Split forward: partial kernel (launch_fwd_split_bf16, d in {64, 128}) and
// the merge of partials (launch_lse_merge, d in {64, 128, 256}, output bf16
// when out_bf16 else float32).
hipError_t launch_fwd_split_bf16(SplitParams p, int d, int causal, hipStream_t stream);
hipError_t launch_lse_merge(const float* Opart, const float* LSEpart, int parts, long long rows, int d, void* O,
                            float* LSE, int out_bf16, hipStream_t stream);
// Keys per tile of the split forward and its waves per workgroup.
constexpr int kSplitBN = 32;
constexpr int split_waves(int d) { return d == 64 ? 4 : 3; }
int split_parts_default(int B, int Hq, int Hkv, int Nq, int Nk, int d);
int split_chunk(int Nk, int parts);
size_t split_workspace_bytes(int B, int Hq, int Nq, int d, int parts);

// Product of non-negative sizes, saturated at LLONG_MAX instead of
// overflowing (limits are then compared against the saturated value).
inline long long sat_mul(long long a, long long b) {
    long long r;
    return __builtin_mul_overflow(a, b, &r) ? 0x7FFFFFFFFFFFFFFFLL : r;
}

// Host state shared by every call: per-device flags and a per-device cache
// of the compute-unit count, both filled once and safe to use from several
// host threads at once (atomics; a race only repeats an idempotent call).
struct DeviceOnce {
    std::atomic<uint64_t> done{0};  // bit i: set on device i
};
// Raises the dynamic-LDS limit of `kern` to `bytes` on the current device,
// once per device.
hipError_t set_max_dynamic_lds(const void* kern, size_t bytes, DeviceOnce& once);
template <typename K>
hipError_t set_max_dynamic_lds(K kern, size_t bytes, DeviceOnce& once) {
    return set_max_dynamic_lds(reinterpret_cast<const void*>(kern), bytes, once);
}
// Compute units of the current device (256 on an MI355X; 256 as well when no
// device can be queried, so host-only size queries stay defined).
int device_cu_count();

}  // namespace fa
