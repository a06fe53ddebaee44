// Split key/value forward and the merge of partial results, bf16 inputs,
// fp32 accumulation, gfx950 matrix cores.
//
// Partial results over blocks of keys combine exactly: each block keeps its
// maximum and its sum of exponentials, and two blocks combine by rescaling
// both to the larger maximum (FlashAttention interview Q&A, app.wittybyte.ai
// "FlashAttention1", softmax answer; the same page lists combining partial
// results computed over different blocks, and incremental attention, among
// what the method enables).  A partial over a key block is kept as
// (O_p normalised by its own sum, LSE_p = m_p + ln l_p); the merge is
//     LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.
//
// fwd_split_kernel<D, CAUSAL>: one wave per (batch, kv head, block of 32
// packed query rows, key range).  Packed row r of kv head g stands for query
// head g*G + r / N_q and query r % N_q (G = H_q / H_kv), so one decoding step
// of a grouped-query head group (N_q = 1) fills G rows of one matrix-core
// block instead of one row of G blocks.  Each wave streams its key range
// through its own double-buffered LDS tiles of 32 keys (direct buffer->LDS
// copies, no barriers: nothing is shared between waves), runs the online
// softmax recurrence of the forward kernel (S^T = K Q^T with one query per
// lane, O^T += V^T P^T with V^T from transposing LDS reads), and writes its
// partial (O_p fp32, LSE_p).  Rows that see no key of the range write
// O_p = 0, LSE_p = -inf.
//
// Causal reading for N_q != N_k: the queries are the last N_q positions of
// the key sequence, so key j is hidden from query i when j > i + N_k - N_q
// (the square rule when N_q = N_k; one query sees every key).
//
// lse_merge_kernel<D, OutT>: one group of D/4 lanes per row, four dims per
// lane; reads every part's LSE, then accumulates the weighted parts.
// lse_merge_wide_kernel<D, OutT>: the same per group of parts, one
// workgroup per row, for many parts over few rows.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <math.h>

namespace fa {

namespace {


// Waves per workgroup (independent of each other) and LDS stages per wave:
// three stages keep two tiles in flight while one is computed, which the
// memory latency of a decoding step needs; at d = 128 three waves of three
// 16 KB stages fill 144 KB of the 160 KB LDS.
template <int D>
struct SplitCfg;
template <>
struct SplitCfg<64> {
    static constexpr int WAVES = split_waves(64), STAGES = 3;
};
template <>
struct SplitCfg<128> {
    static constexpr int WAVES = split_waves(128), STAGES = 3;
};

template <int D>
constexpr int split_tile_bytes() {
    return kSplitBN * D * 2;  // one tile of K (or of V)
}
template <int D>
constexpr size_t split_lds_bytes() {
    return size_t(SplitCfg<D>::WAVES) * SplitCfg<D>::STAGES * 2 * split_tile_bytes<D>();
}

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations
// (here: buffer->LDS copies) still in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wave-wide max of an int (butterfly over the 64 lanes).
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
    return x;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(SplitCfg<D>::WAVES * 64) void fwd_split_kernel(SplitParams p) {
    constexpr int BN = kSplitBN;
    constexpr int NW = SplitCfg<D>::WAVES, NST = SplitCfg<D>::STAGES;
    constexpr int TB = split_tile_bytes<D>();
    constexpr int PIECES = TB / 1024;  // 1 KB copy pieces per matrix per tile
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;

    // blockIdx.x -> (unit = batch x kv head, row block, group of NW parts)
    const int units = p.B * p.Hkv;
    int id = blockIdx.x;
    const int unit = id % units;
    id /= units;
    const int rb = id % p.nrb;
    const int part = (id / p.nrb) * NW + w;
    if (part >= p.parts) return;  // nothing is shared between waves: no barrier to keep

    const int b = unit / p.Hkv, g = unit - (unit / p.Hkv) * p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int Nq = p.Nq, Nk = p.Nk;
    const int k_begin = part * p.chunk;
    const int k_end = min(Nk, k_begin + p.chunk);

    // Packed row of this lane and the last key it may see.
    const int r = rb * 32 + l32;
    const bool row_ok = r < G * Nq;
    const int hq = g * G + (row_ok ? r / Nq : 0);
    const int qi = row_ok ? r - (r / Nq) * Nq : 0;
    int key_lim = CAUSAL ? min(Nk - 1, qi + Nk - Nq) : Nk - 1;
    if (!row_ok) key_lim = -1;
    const int k_stop = min(k_end, wave_max(key_lim) + 1);  // uniform
    const int ntiles = k_stop > k_begin ? (k_stop - k_begin + BN - 1) / BN : 0;

    const size_t kvoff = size_t(b * p.Hkv + g) * size_t(Nk) * D;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;
    unsigned char* base = smem_raw + size_t(w) * NST * 2 * TB;

    // Per-lane in-tile byte offsets of the pieces this lane copies (slab
    // layouts of fa_device.hpp: K slabs for row reads, V slabs for
    // transposing reads).
    uint32_t koff[PIECES], voff[PIECES];
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
        int rr, e0;
        kslab_slot<BN>(64 * i + lane, rr, e0);
        koff[i] = uint32_t(2 * (rr * D + e0));
        vslab_slot<BN>(64 * i + lane, rr, e0);
        voff[i] = uint32_t(2 * (rr * D + e0));
    }
    auto issue = [&](int key0, int stage) {
        unsigned char* st = base + stage * 2 * TB;
        const uint32_t bytes = uint32_t(Nk - key0) * uint32_t(D * 2);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kh + size_t(key0) * D, bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vh + size_t(key0) * D, bytes);
        const uint32_t last = uint32_t(Nk - 1 - key0);  // rows past N_k read row N_k - 1 (masked later)
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const uint32_t rk = koff[i] / (2 * D), rv = voff[i] / (2 * D);
            const uint32_t ok = min(rk, last) * (2 * D) + koff[i] % (2 * D);
            const uint32_t ov = min(rv, last) * (2 * D) + voff[i] % (2 * D);
            buf16_to_lds(kr, ok, st + 1024 * i);
            buf16_to_lds(vr, ov, st + TB + 1024 * i);
        }
    };
    // Q rows of this lane as MFMA B operands (qmode 1 negates, 2 zeroes),
    // loaded before the first copies so that waiting for them does not wait
    // for the copies.
    bf16x8 qreg[D / 16];
    {
        const bf16* Qr = static_cast<const bf16*>(p.Q) + (size_t(b * p.Hq + hq) * Nq + qi) * D;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            u32x4 v = u32x4{0, 0, 0, 0};
            if (row_ok && p.qmode != 2) v = ld16(Qr + 16 * cc + 8 * hi);
            if (p.qmode == 1) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qreg[cc] = as_bf16x8(v);
        }
    }

#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
        if (t < ntiles) issue(k_begin + t * BN, t);

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    // A finite floor for the running max: a row that has seen no key yet
    // keeps factors exp2(m_old - m_new) well defined (1, or 0 on its first
    // visible key) and exp2(c s - m) = 0 for its masked scores.
    float m = -3.0e38f;
    float l = 0.f;
    const float c = p.scale_log2;  // > 0
    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    static_assert(NST == 3, "the waits below are written for three stages");
    for (int t = 0; t < ntiles; ++t) {
        // The stage of tile t-1 was consumed in the previous iteration:
        // refill it with tile t+NST-1.
        if (t + NST - 1 < ntiles) issue(k_begin + (t + NST - 1) * BN, (t + NST - 1) % NST);
        // Tile t has landed once only the copies of the tiles issued after
        // it (t+1 .. t+NST-1, those that exist) are in flight.
        const int after = min(NST - 1, ntiles - 1 - t);
        if (after == 2) wait_vmem_n<4 * PIECES>();
        else if (after == 1) wait_vmem_n<2 * PIECES>();
        else wait_vmem();
        const int stage = t % NST;
        const bf16* Ks = reinterpret_cast<const bf16*>(base + stage * 2 * TB);
        const bf16* Vs = reinterpret_cast<const bf16*>(base + stage * 2 * TB + TB);
        const int key0 = k_begin + t * BN;

        // S^T (32 keys x 32 rows): s[r] = score(key key0 + 8(r/4) + 4hi + r%4, row of this lane)
        f32x16 s = f32x16{};
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc)
            s = mfma_32x32x16(as_bf16x8(lds16(Ks + kslab_off<BN>(l32, 16 * cc + 8 * hi))), qreg[cc], s);
        // keys past this row's limit (causal, N_k, invalid rows) are hidden
        {
            const int lim = key_lim - key0 - 4 * hi;
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) s[rr] = (8 * (rr >> 2) + (rr & 3) > lim) ? -INFINITY : s[rr];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
        mx = half_swap_max(mx) * c;
        if (__any(mx > m)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        }
        float e[16];
        float rs = 0.f;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            e[rr] = fast_exp2(fmaf(s[rr], c, -m));
            rs += e[rr];
        }
        l += rs;
        const bf16x8 pb0 = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        const bf16x8 pb1 = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
        // O^T += V^T P^T; contraction slot (cc, hi, sl) <-> key 16cc + 8(sl/4) + 4hi + sl%4
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int key = 16 * cc + trow;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const bf16x4 v0 = lds_read_tr(Vs + vslab_off<BN>(key, db * 32 + tcol));
                const bf16x4 v1 = lds_read_tr(Vs + vslab_off<BN>(key + 8, db * 32 + tcol));
                o[db] = mfma_32x32x16(cat(v0, v1), cc ? pb1 : pb0, o[db]);
            }
        }
    }
    wait_vmem();  // no copy into LDS may outlive the wave

    // Partial output: O_p = o / l (fp32), LSE_p = ln2 (m + log2 l); -inf when
    // the row saw no key of this range.
    const float lt = half_swap_sum(l);
    if (row_ok) {
        const size_t row = size_t(b * p.Hq + hq) * Nq + qi;
        const size_t rows = size_t(p.B) * p.Hq * Nq;
        float* Orow = p.Opart + (size_t(part) * rows + row) * D;
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = f32x4{o[db][4 * j + 0] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                                      o[db][4 * j + 3] * inv};
                *reinterpret_cast<f32x4*>(Orow + db * 32 + 8 * j + 4 * hi) = v;
            }
        }
        if (hi == 0) p.LSEpart[size_t(part) * rows + row] = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    }
}

// Merge of `parts` partial results per row: O_parts fp32 [parts][rows][D],
// LSE_parts fp32 [parts][rows] -> O [rows][D] (OutT), LSE [rows] fp32.
// One wave per block (64 / (D/4) rows); the loops over the parts are
// unrolled so that several loads are in flight (few rows, many parts is the
// decoding case, where this kernel is latency-bound).
constexpr int kMergeThreads = 64;
template <int D, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const float* __restrict__ Op,
                                                                  const float* __restrict__ Lp, int parts,
                                                                  long long rows, OutT* __restrict__ O,
                                                                  float* __restrict__ LSE) {
    constexpr int TPR = D / 4;                   // lanes per row, four dims each
    constexpr int RPB = kMergeThreads / TPR > 0 ? kMergeThreads / TPR : 1;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int t = threadIdx.x % TPR;
    if (row >= rows) return;
    float M = -INFINITY;
#pragma unroll 8
    for (int q = 0; q < parts; ++q) M = fmaxf(M, Lp[(long long)q * rows + row]);
    float tot = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll 8
        for (int q = 0; q < parts; ++q) {
            const float lq = Lp[(long long)q * rows + row];
            const f32x4 v = *reinterpret_cast<const f32x4*>(Op + ((long long)q * rows + row) * D + 4 * t);
            const float wq = lq == -INFINITY ? 0.f : expf(lq - M);  // empty parts hold O_p = 0
            tot += wq;
            acc += wq * v;
        }
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    OutT* orow = O + row * D + 4 * t;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = OutT(acc[e] * inv);
    if (t == 0 && LSE != nullptr) LSE[row] = tot > 0.f ? M + logf(tot) : -INFINITY;
}

// Many parts (decoding steps split over many key ranges, few rows): one
// workgroup of 256 threads per row; the row's parts are dealt to 256 / (D/4)
// lane groups, each group merges its own parts as above (its own max, sum
// and weighted output), and the groups' partials are merged through LDS
// with the same rule: M = max_g M_g, sum = sum_g sum_g e^{M_g - M},
// O = sum_g acc_g e^{M_g - M} / sum.
constexpr int kMergeWideThreads = 256;
template <int D, typename OutT>
__global__ __launch_bounds__(kMergeWideThreads) void lse_merge_wide_kernel(const float* __restrict__ Op,
                                                                           const float* __restrict__ Lp, int parts,
                                                                           long long rows, OutT* __restrict__ O,
                                                                           float* __restrict__ LSE) {
    constexpr int TPR = D / 4;                     // lanes per part group, four dims each
    constexpr int PG = kMergeWideThreads / TPR;    // part groups
    __shared__ float sm[PG], ssum[PG];
    __shared__ f32x4 sacc[PG][TPR];
    const long long row = blockIdx.x;
    const int t = threadIdx.x % TPR, g = threadIdx.x / TPR;
    float m = -INFINITY;
    for (int q = g; q < parts; q += PG) m = fmaxf(m, Lp[(long long)q * rows + row]);
    float tot = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY) {
        for (int q = g; q < parts; q += PG) {
            const float lq = Lp[(long long)q * rows + row];
            const f32x4 v = *reinterpret_cast<const f32x4*>(Op + ((long long)q * rows + row) * D + 4 * t);
            const float wq = lq == -INFINITY ? 0.f : expf(lq - m);  // empty parts hold O_p = 0
            tot += wq;
            acc += wq * v;
        }
    }
    if (t == 0) {
        sm[g] = m;
        ssum[g] = tot;
    }
    sacc[g][t] = acc;
    __syncthreads();
    if (g != 0) return;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < PG; ++k) M = fmaxf(M, sm[k]);
    float sum = 0.f;
    f32x4 out = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int k = 0; k < PG; ++k) {
            const float f = sm[k] == -INFINITY ? 0.f : expf(sm[k] - M);
            sum += ssum[k] * f;
            out += f * sacc[k][t];
        }
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    OutT* orow = O + row * D + 4 * t;
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[e] = OutT(out[e] * inv);
    if (t == 0 && LSE != nullptr) LSE[row] = sum > 0.f ? M + logf(sum) : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_split_t(SplitParams p, hipStream_t stream) {
    auto kern = fwd_split_kernel<D, CAUSAL>;
    constexpr size_t lds = split_lds_bytes<D>();
    static DeviceOnce attr;
    hipError_t e = set_max_dynamic_lds(kern, lds, attr);
    if (e != hipSuccess) return e;
    constexpr int NW = SplitCfg<D>::WAVES;
    const long long blocks = (long long)p.B * p.Hkv * p.nrb * ((p.parts + NW - 1) / NW);
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(NW * 64), lds, stream, p);
    return hipGetLastError();
}

template <int D, typename OutT>
hipError_t launch_merge_t(const float* Op, const float* Lp, int parts, long long rows, void* O, float* LSE,
                          hipStream_t stream) {
    constexpr int TPR = D / 4;
    if (parts >= 8 && rows <= (1LL << 16)) {
        // many parts over few rows: one workgroup per row (the narrow kernel would
        // leave each lane a long chain of dependent loads)
        hipLaunchKernelGGL((lse_merge_wide_kernel<D, OutT>), dim3(unsigned(rows)), dim3(kMergeWideThreads), 0,
                           stream, Op, Lp, parts, rows, static_cast<OutT*>(O), LSE);
        return hipGetLastError();
    }
    constexpr int RPB = kMergeThreads / TPR > 0 ? kMergeThreads / TPR : 1;
    constexpr int THREADS = RPB * TPR;  // 64, or one row of 64 lanes at d = 256
    const long long blocks = (rows + RPB - 1) / RPB;
    hipLaunchKernelGGL((lse_merge_kernel<D, OutT>), dim3(unsigned(blocks)), dim3(THREADS), 0, stream, Op, Lp, parts,
                       rows, static_cast<OutT*>(O), LSE);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_split_bf16(SplitParams p, int d, int causal, hipStream_t stream) {
    if (p.scale_log2 > 0.f) {
        p.qmode = 0;
    } else if (p.scale_log2 < 0.f) {
        p.qmode = 1;
        p.scale_log2 = -p.scale_log2;
    } else {
        p.qmode = 2;
        p.scale_log2 = 1.f;
    }
    p.chunk = split_chunk(p.Nk, p.parts);
    p.nrb = ((p.Hq / p.Hkv) * p.Nq + 31) / 32;
    switch (d) {
        case 64: return causal ? launch_split_t<64, true>(p, stream) : launch_split_t<64, false>(p, stream);
        case 128: return causal ? launch_split_t<128, true>(p, stream) : launch_split_t<128, false>(p, stream);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_lse_merge(const float* Op, const float* Lp, int parts, long long rows, int d, void* O, float* LSE,
                            int out_bf16, hipStream_t stream) {
    switch (d) {
        case 64:
            return out_bf16 ? launch_merge_t<64, bf16>(Op, Lp, parts, rows, O, LSE, stream)
                            : launch_merge_t<64, float>(Op, Lp, parts, rows, O, LSE, stream);
        case 128:
            return out_bf16 ? launch_merge_t<128, bf16>(Op, Lp, parts, rows, O, LSE, stream)
                            : launch_merge_t<128, float>(Op, Lp, parts, rows, O, LSE, stream);
        case 256:
            return out_bf16 ? launch_merge_t<256, bf16>(Op, Lp, parts, rows, O, LSE, stream)
                            : launch_merge_t<256, float>(Op, Lp, parts, rows, O, LSE, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace fa
