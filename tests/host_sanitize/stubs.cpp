// Host-only stand-ins for everything the C ABI calls below it: the kernel
// launchers, the device scratch buffer and the few HIP runtime calls.  With
// these, fa_api.cpp and fa_host.cpp build with a host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer, and every validation path
// runs without a device.  Each launcher checks that the arguments it would
// hand to a kernel are within what the kernels assume, and counts the call.
#include "fa.h"
#include "fa_internal.h"

#include <cmath>
#include <cstdio>
#include <cstdlib>

int g_launches = 0;

namespace {

void require(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "launcher precondition failed: %s\n", what);
        std::abort();
    }
}

void check_window(int wl, int wr) {
    require(wl >= 0 && wl <= fa::kUnbounded, "0 <= wl <= kUnbounded");
    require(wr >= 0 && wr <= fa::kUnbounded, "0 <= wr <= kUnbounded");
}

template <typename P>
void check_common(const P& p) {
    require(p.B >= 1 && p.N >= 1, "B, N >= 1 past the nothing-to-do exit");
    require(p.Hkv >= 1 && p.Hq >= p.Hkv && p.Hq % p.Hkv == 0, "head grouping");
    require(std::isfinite(p.scale_log2), "finite scale");
    require(p.Q && p.K && p.V, "inputs non-null");
    if (p.cu) require(p.total >= 0, "packed total");
    if (p.bmask) require(p.nb == (p.N + fa::kSparseBlock - 1) / fa::kSparseBlock, "block map size");
    require(p.drop_t8 >= 0 && p.drop_t8 <= 255, "dropout threshold");
}

}  // namespace

namespace fa {

hipError_t launch_fwd_bf16(FwdParams p, int d, int causal, hipStream_t) {
    check_common(p);
    require(d == 64 || d == 128 || d == 256, "bf16 head dim");
    require(p.O != nullptr, "O non-null");
    if (causal) check_window(p.wl, p.wr);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_fwd_f32(FwdParams p, int d, int causal, hipStream_t) {
    check_common(p);
    require(d == 64 || d == 128 || d == 256, "f32 head dim");
    if (causal) check_window(p.wl, p.wr);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_bwd_bf16(BwdParams p, int d, int causal, hipStream_t) {
    check_common(p);
    require(d == 64 || d == 128, "bf16 backward head dim");
    require(p.O && p.dO && p.LSE && p.dQ && p.dK && p.dV && p.Drow, "backward pointers");
    require(p.hsplit >= 1 && (p.Hq / p.Hkv) % p.hsplit == 0, "query-head split divides the group");
    if (p.hsplit > 1) require(p.dk_part && p.dv_part && p.part_stride > 0, "split partials");
    if (causal) check_window(p.wl, p.wr);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_bwd_f32(BwdParams p, int d, int causal, hipStream_t) {
    check_common(p);
    require(d == 64 || d == 128 || d == 256, "f32 backward head dim");
    require(p.hsplit == 1, "no split in float32");
    if (causal) check_window(p.wl, p.wr);
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_fwd_split_bf16(SplitParams p, int d, int, hipStream_t) {
    require(p.B >= 1 && p.Nq >= 1 && p.Nk >= 1, "split sizes");
    require(p.parts >= 1 && p.parts <= FA_MAX_SPLITS, "split parts");
    require(d == 64 || d == 128, "split head dim");
    require(p.Opart && p.LSEpart, "split partials");
    ++g_launches;
    return hipSuccess;
}

hipError_t launch_lse_merge(const float* Opart, const float* LSEpart, int parts, long long rows, int d, void* O,
                            float*, int, hipStream_t) {
    require(Opart && LSEpart && O, "merge pointers");
    require(parts >= 1 && parts <= FA_MAX_SPLITS && rows >= 1, "merge sizes");
    require(d == 64 || d == 128 || d == 256, "merge head dim");
    ++g_launches;
    return hipSuccess;
}

void* noalloc_scratch(hipError_t& err) {
    alignas(256) static unsigned char host_stand_in[256];  // never dereferenced by the stub launchers
    err = hipSuccess;
    return host_stand_in;
}

}  // namespace fa

// HIP runtime calls made by the C ABI itself: no device is present.
extern "C" {
hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) { return hipSuccess; }
}
