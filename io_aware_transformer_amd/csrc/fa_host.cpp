// Host-side size and decomposition rules shared by the C ABI and the
// launchers: workspace sizes of the backward and of the split forward, the
// query-head split of a grouped backward and the key ranges of the split
// forward.  Plain C++ with no device code, so the C ABI and these rules also
// build with a host compiler alone (the sanitizer build of the validation
// paths does).
#include "fa_internal.h"

namespace fa {

size_t bwd_workspace_bytes(int Hq, long long rows) {
    const size_t d_bytes = size_t(Hq) * size_t(rows) * sizeof(float);
    return (d_bytes + 255) / 256 * 256;
}

int bwd_hsplit(int B, int Hq, int Hkv, int N) {
    // dK/dV workgroups of 128 keys (the d = 64 kernel takes 256; the split is
    // sized on 128 so the workspace does not depend on the kernel): aim for
    // two workgroups per compute unit.
    const int G = Hq / Hkv;
    const long long wgs = (long long)((N + 127) / 128) * B * Hkv;
    const long long want = 2LL * device_cu_count();
    int s = 1;
    while (wgs * s < want && G % (2 * s) == 0) s *= 2;
    return s;
}

size_t bwd_workspace_bytes_split(int B, int Hq, int Hkv, int N, int d) {
    size_t bytes = bwd_workspace_bytes(Hq, (long long)B * N);
    const int s = bwd_hsplit(B, Hq, Hkv, N);
    if (s > 1) {
        const size_t part = (size_t(s) * B * Hkv * N * d * sizeof(float) + 255) / 256 * 256;
        bytes += 2 * part;
    }
    return bytes;
}

int split_chunk(int Nk, int parts) {
    const int per = (Nk + parts - 1) / parts;
    return (per + kSplitBN - 1) / kSplitBN * kSplitBN;
}

int split_parts_default(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    // One workgroup per compute unit (split_waves(d) waves each: the LDS
    // holds one), with at least four 32-key tiles per part.
    const int nw = split_waves(d);
    const long long rows = (long long)(Hq / Hkv) * Nq;
    const long long waves = sat_mul(sat_mul(B, Hkv), (rows + 31) / 32);
    long long parts = ((long long)device_cu_count() * nw + waves - 1) / waves;
    const long long max_parts = ((long long)Nk + 4 * kSplitBN - 1) / (4 * kSplitBN);
    if (parts > max_parts) parts = max_parts;
    if (parts < 1) parts = 1;
    return int(parts);
}

size_t split_workspace_bytes(int B, int Hq, int Nq, int d, int parts) {
    const size_t rows = size_t(B) * Hq * Nq;
    const size_t o = size_t(parts) * rows * d * sizeof(float);
    const size_t lse = size_t(parts) * rows * sizeof(float);
    return (o + 255) / 256 * 256 + (lse + 255) / 256 * 256;
}

}  // namespace fa
