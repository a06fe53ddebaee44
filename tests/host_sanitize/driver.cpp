// Drives every validation path of the C ABI on the host: boundary and
// out-of-range values of each argument, then a seeded random mix of them.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer (any report
// aborts); exits 0 when every call returned a defined status, valid calls
// reached a launcher and rejected ones launched nothing.
#include "fa.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>
#include <limits>

extern int g_launches;

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
    if (!ok) {
        std::fprintf(stderr, "FAIL line %d: %s\n", line, what);
        ++failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

bool defined_status(int st) { return st <= FA_OK && st >= FA_ERR_ARG; }

// Fake device addresses: never dereferenced (the launchers are stand-ins).
void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);
void* const MIS = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);
const float* const PF = static_cast<const float*>(P);
const int* const PI = static_cast<const int*>(P);
const unsigned char* const PB = static_cast<const unsigned char*>(P);

const int kInts[] = {INT_MIN, -2, -1, 0, 1, 2, 3, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                     FA_MAX_HEADS, FA_MAX_HEADS + 1, FA_SPARSE_MAX_N, FA_SPARSE_MAX_N + 1,
                     FA_MAX_N, FA_MAX_N + 1, INT_MAX - 1, INT_MAX};
const float kScales[] = {0.125f, 1.0f, -0.5f, 0.0f, -0.0f, 1e-45f, 3e38f,
                         std::numeric_limits<float>::infinity(), -std::numeric_limits<float>::infinity(),
                         std::numeric_limits<float>::quiet_NaN()};
const float kProbs[] = {0.0f, 0.1f, 0.5f, 0.996f, 0.999f, 1.0f, -0.1f, 2.0f,
                        std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::infinity()};
const size_t kSizes[] = {0, 1, 255, 256, size_t(1) << 30, SIZE_MAX};

uint64_t rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // splitmix64
    uint64_t z = (rng += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
template <typename T, size_t n>
T pick(const T (&a)[n]) {
    return a[next() % n];
}
int small() { return int(next() % 5); }        // 0 .. 4
int pick_d() { return (next() & 1) ? (64 << (next() % 3)) : pick(kInts); }
int pick_bool() { return (next() % 4) ? int(next() & 1) : pick(kInts); }
void* pick_ptr() {
    const int r = int(next() % 8);
    return r == 0 ? nullptr : r == 1 ? MIS : P;
}

// A call that returned FA_OK may have launched; any other status must not.
void check_call(int st, int launches_before) {
    EXPECT(defined_status(st));
    if (st != FA_OK) EXPECT(g_launches == launches_before);
}

void run_one_random() {
    const int B = (next() & 1) ? small() : pick(kInts);
    const int Hkv = (next() & 1) ? 1 + small() : pick(kInts);
    const int Hq = (next() & 1) && Hkv > 0 && Hkv < 1000 ? Hkv * (1 + small()) : pick(kInts);
    const int N = (next() & 1) ? int(next() % 5000) : pick(kInts);
    const int d = pick_d();
    const float sc = pick(kScales);
    const int causal = pick_bool();
    const int dtype = (next() % 4) ? int(next() & 1) : pick(kInts);
    void* q = pick_ptr();
    const size_t ws_bytes = (next() & 1) ? fa_bwd_workspace_size(B, Hq, Hkv, N, d, dtype) : pick(kSizes);
    const int before = g_launches;
    int st = 0;
    switch (next() % 12) {
        case 0: st = fa_fwd(q, P, P, P, static_cast<float*>(pick_ptr()), B, Hq, Hkv, N, d, sc, causal, dtype, nullptr); break;
        case 1:
            st = fa_bwd(q, P, P, P, P, PF, P, P, pick_ptr(), pick_ptr(), ws_bytes, B, Hq, Hkv, N, d, sc, causal, dtype,
                        nullptr);
            break;
        case 2:
            st = fa_fwd_window(q, P, P, P, nullptr, B, Hq, Hkv, N, d, sc, pick(kInts), pick(kInts), dtype, nullptr);
            break;
        case 3:
            st = fa_bwd_window(q, P, P, P, P, PF, P, P, P, pick_ptr(), ws_bytes, B, Hq, Hkv, N, d, sc, pick(kInts),
                               pick(kInts), dtype, nullptr);
            break;
        case 4:
            st = fa_fwd_blocksparse(q, P, P, P, nullptr, (next() & 1) ? PB : nullptr, B, Hq, Hkv, N, d, sc, causal,
                                    dtype, nullptr);
            break;
        case 5:
            st = fa_bwd_blocksparse(q, P, P, P, P, PF, P, P, P, pick_ptr(), ws_bytes, PB, B, Hq, Hkv, N, d, sc, causal,
                                    dtype, nullptr);
            break;
        case 6:
            st = fa_fwd_dropout(q, P, P, P, nullptr, B, Hq, Hkv, N, d, sc, causal, pick(kProbs), next(),
                                unsigned(next()), dtype, nullptr);
            break;
        case 7:
            st = fa_bwd_dropout(q, P, P, P, P, PF, P, P, P, pick_ptr(), ws_bytes, B, Hq, Hkv, N, d, sc, causal,
                                pick(kProbs), next(), unsigned(next()), dtype, nullptr);
            break;
        case 8: {
            const int total = (next() & 1) ? int(next() % 9000) : pick(kInts);
            const int maxlen = (next() & 1) ? int(next() % 9000) : pick(kInts);
            if (next() & 1) {
                st = fa_fwd_varlen(q, P, P, P, nullptr, (next() & 1) ? PI : nullptr, B, total, maxlen, Hq, Hkv, d, sc,
                                   causal, dtype, nullptr);
            } else {
                const size_t w = (next() & 1) ? fa_bwd_varlen_workspace_size(total, Hq, Hkv, d, dtype) : pick(kSizes);
                st = fa_bwd_varlen(q, P, P, P, P, PF, P, P, P, pick_ptr(), w, PI, B, total, maxlen, Hq, Hkv, d, sc,
                                   causal, dtype, nullptr);
            }
            break;
        }
        case 9: {
            const int Nq = (next() & 1) ? 1 + small() : pick(kInts);
            const int splits = (next() & 1) ? small() : pick(kInts);
            const size_t w = (next() & 1) ? fa_fwd_split_workspace_size(B, Hq, Hkv, Nq, N, d, splits, dtype)
                                          : pick(kSizes);
            (void)fa_fwd_split_parts(B, Hq, Hkv, Nq, N, d, splits);
            st = fa_fwd_split(q, P, P, P, nullptr, B, Hq, Hkv, Nq, N, d, sc, causal, splits, pick_ptr(), w, dtype,
                              nullptr);
            break;
        }
        case 10: {
            const long long rows = (next() & 1) ? (long long)(next() % 100000) : (long long)pick(kInts);
            st = fa_lse_merge(static_cast<const float*>(pick_ptr()), PF, (next() & 1) ? small() : pick(kInts), rows, d,
                              P, nullptr, dtype, nullptr);
            break;
        }
        default:
            st = fa_bwd_noalloc(q, P, P, P, P, PF, P, P, P, B, Hq, Hkv, N, d, sc, causal, dtype, nullptr);
            break;
    }
    check_call(st, before);
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? std::atol(argv[1]) : 1000000;
    if (argc > 2) rng = std::strtoull(argv[2], nullptr, 0);

    // Fixed expectations.
    int before = g_launches;
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, 300, 128, 0.1f, 1, FA_BF16, nullptr) == FA_OK);
    EXPECT(g_launches == before + 1);
    EXPECT(fa_fwd(MIS, P, P, P, nullptr, 2, 4, 2, 300, 128, 0.1f, 1, FA_BF16, nullptr) == FA_ERR_ALIGN);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 3, 300, 128, 0.1f, 1, FA_BF16, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, FA_MAX_N + 1, 128, 0.1f, 1, FA_BF16, nullptr) == FA_ERR_SHAPE);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, 300, 96, 0.1f, 1, FA_BF16, nullptr) == FA_ERR_HEADDIM);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, 300, 128, NAN, 1, FA_BF16, nullptr) == FA_ERR_ARG);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, 300, 128, 0.1f, 2, FA_BF16, nullptr) == FA_ERR_ARG);
    EXPECT(fa_fwd(P, P, P, P, nullptr, 2, 4, 2, 300, 128, 0.1f, 1, 7, nullptr) == FA_ERR_DTYPE);
    EXPECT(fa_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 4, 2, 300, 128, 0.1f, 1, FA_BF16, nullptr) == FA_OK);
    // windows past the sequence are the unbounded case; INT_MAX bounds are accepted
    for (int wl : {-1, 0, 5, 299, 300, INT_MAX})
        for (int wr : {-1, 0, 5, 299, 300, INT_MAX})
            EXPECT(fa_fwd_window(P, P, P, P, nullptr, 1, 2, 2, 300, 64, 0.1f, wl, wr, FA_BF16, nullptr) == FA_OK);
    EXPECT(fa_fwd_window(P, P, P, P, nullptr, 1, 2, 2, 300, 64, 0.1f, -2, 0, FA_BF16, nullptr) == FA_ERR_ARG);
    EXPECT(fa_fwd_window(P, P, P, P, nullptr, 1, 2, 2, 300, 64, 0.1f, INT_MIN, 0, FA_BF16, nullptr) == FA_ERR_ARG);
    // backward workspace: exactly the size query passes, one byte less fails
    for (int Hkv : {1, 2, 8}) {
        const size_t need = fa_bwd_workspace_size(1, 8, Hkv, 1000, 128, FA_BF16);
        EXPECT(need > 0);
        EXPECT(fa_bwd(P, P, P, P, P, PF, P, P, P, P, need, 1, 8, Hkv, 1000, 128, 0.1f, 1, FA_BF16, nullptr) == FA_OK);
        EXPECT(fa_bwd(P, P, P, P, P, PF, P, P, P, P, need - 1, 1, 8, Hkv, 1000, 128, 0.1f, 1, FA_BF16, nullptr) ==
               FA_ERR_WORKSPACE);
    }
    EXPECT(fa_bwd(P, P, P, P, P, PF, P, P, P, P, SIZE_MAX, 1, 8, 2, 1000, 256, 0.1f, 1, FA_BF16, nullptr) ==
           FA_ERR_UNSUPPORTED);
    // the buffer-free backward's row limit
    EXPECT(fa_bwd_noalloc(P, P, P, P, P, PF, P, P, P, 1, 16, 16, FA_NOALLOC_MAX_ROWS / 16, 64, 0.1f, 1, FA_BF16,
                          nullptr) == FA_OK);
    EXPECT(fa_bwd_noalloc(P, P, P, P, P, PF, P, P, P, 1, 16, 16, FA_NOALLOC_MAX_ROWS / 16 + 1, 64, 0.1f, 1, FA_BF16,
                          nullptr) == FA_ERR_WORKSPACE);
    // dropout probability rounding to 256 / 256 is rejected
    EXPECT(fa_fwd_dropout(P, P, P, P, nullptr, 1, 2, 2, 64, 64, 0.1f, 1, 0.999f, 1, 0, FA_BF16, nullptr) == FA_ERR_ARG);
    EXPECT(fa_fwd_dropout(P, P, P, P, nullptr, 1, 2, 2, 64, 64, 0.1f, 1, 0.998f, 1, 0, FA_BF16, nullptr) == FA_OK);
    // block-sparse length limit (the kernels' tile lists)
    EXPECT(fa_fwd_blocksparse(P, P, P, P, nullptr, PB, 1, 1, 1, FA_SPARSE_MAX_N + 1, 64, 0.1f, 0, FA_BF16, nullptr) ==
           FA_ERR_UNSUPPORTED);
    // status strings are never null
    for (int s = -20; s <= 5; ++s) EXPECT(fa_status_str(s) != nullptr);
    EXPECT(fa_version() > 0);

    // Boundary value of every integer argument of fa_fwd / fa_bwd in turn.
    for (int which = 0; which < 4; ++which)
        for (int v : kInts) {
            int a[4] = {2, 4, 2, 300};
            a[which] = v;
            before = g_launches;
            int st = fa_fwd(P, P, P, P, nullptr, a[0], a[1], a[2], a[3], 64, 0.1f, 1, FA_BF16, nullptr);
            check_call(st, before);
            const size_t w = fa_bwd_workspace_size(a[0], a[1], a[2], a[3], 64, FA_BF16);
            before = g_launches;
            st = fa_bwd(P, P, P, P, P, PF, P, P, P, P, w, a[0], a[1], a[2], a[3], 64, 0.1f, 1, FA_BF16, nullptr);
            check_call(st, before);
        }

    for (long i = 0; i < iters; ++i) run_one_random();

    std::printf("%ld random calls, %d launches, %d failures\n", iters, g_launches, failures);
    return failures == 0 ? 0 : 1;
}
