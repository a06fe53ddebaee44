// Forward pass, bf16 inputs, fp32 accumulation, gfx950 matrix cores.
//
// Method: exact attention evaluated tile by tile with the online softmax
// recurrence (FlashAttention interview Q&A, app.wittybyte.ai
// "FlashAttention1", softmax answer: running max m and running sum l, the
// old sum rescaled by exp(m_old - m_new)); the running output is rescaled by
// the same factor (deep-dive page "Flash attention: fast and
// memory-efficient exact attention with IO-awareness", "Intuition").  The
// score tile lives only in registers; only O and the per-row LSE reach HBM.
//
// Work decomposition ("The Future of AI: How FlashAttention Revolutionizes
// Deep Learning", "FlashAttention-2: Enhanced Performance": parallel over
// sequence length as well as batch and heads; queries split across warps
// while keys/values are shared): one workgroup of 4 waves per
// (batch, query head, block of 128 query rows); each wave owns 32 query
// rows; K/V tiles of BN keys are staged in LDS (double-buffered through
// registers) and read by all four waves.
//
// Per wave and 32-key block, in the layouts of fa_device.hpp:
//   S^T (32 keys x 32 queries) = K_blk . Q^T     A = K rows (LDS), B = Q (regs)
//   lane l then holds one query (l % 32) and 16 of its keys, so the row
//   max/sum are in-lane plus one v_permlane32_swap across the halves.
//   O^T (d x 32 queries) += V^T . P^T            A = V^T via ds_read_b64_tr_b16,
//   B = P^T straight from the score registers (the key order inside the
//   contraction is permuted consistently on both operands).
// Scores are scaled by scale*log2(e) so the exponentials are exp2 (v_exp_f32);
// LSE is converted back to natural log at the end.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <math.h>

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;  // query rows per workgroup

template <int D>
struct FwdTile;
template <>
struct FwdTile<64> {
    static constexpr int BN = 64;
};
template <>
struct FwdTile<128> {
    static constexpr int BN = 64;
};
template <>
struct FwdTile<256> {
    static constexpr int BN = 32;
};

template <int D>
constexpr size_t fwd_lds_bytes() {
    return size_t(2) /*stages*/ * 2 /*K,V*/ * FwdTile<D>::BN * D * sizeof(bf16);
}

// Workgroup id -> (query block, batch, head).  Heaviest causal query blocks
// are issued first.  Workgroups are dealt round-robin to the 8 XCDs; when
// the number of (batch, head) units is a multiple of 8, consecutive units
// are remapped onto one XCD so heads sharing K/V share that XCD's L2.
__device__ __forceinline__ void fwd_decompose(int id, int units, int nqb, int Hq, bool causal, int& qb, int& b,
                                              int& h) {
    const int slot = id / units;
    const int u = id - slot * units;
    qb = causal ? nqb - 1 - slot : slot;
    const int unit = (units % 8 == 0) ? (u & 7) * (units >> 3) + (u >> 3) : u;
    b = unit / Hq;
    h = unit - b * Hq;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(FwdParams p) {
    constexpr int BN = FwdTile<D>::BN;
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    constexpr int TILE = BN * D;
    constexpr int NLD = BN * CPR / 256;  // chunks per thread per tile and matrix
    static_assert(NLD >= 1 && (BN * CPR) % 256 == 0, "tile must split evenly over 256 threads");
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int N = p.N;

    int qb, b, h;
    fwd_decompose(blockIdx.x, p.B * p.Hq, p.nqb, p.Hq, CAUSAL, qb, b, h);
    const int g = h / (p.Hq / p.Hkv);
    const size_t qoff = size_t(b * p.Hq + h) * size_t(N) * D;
    const size_t kvoff = size_t(b * p.Hkv + g) * size_t(N) * D;
    const bf16* __restrict__ Qh = static_cast<const bf16*>(p.Q) + qoff;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;
    bf16* __restrict__ Oh = static_cast<bf16*>(p.O) + qoff;

    const int q0 = qb * kBM;
    const int wq0 = q0 + 32 * w;  // first query row of this wave
    const int qrow = wq0 + l32;   // the query row this lane works for

    // Q tile of this wave as the MFMA B operand: Q[qrow][16c + 8hi .. +7].
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        if (qrow < N) qreg[c] = as_bf16x8(ld16(Qh + size_t(qrow) * D + 16 * c + 8 * hi));
        else qreg[c] = bf16x8{};
    }

    const int kend = CAUSAL ? min(N, q0 + kBM) : N;
    const int ntiles = (kend + BN - 1) / BN;

    u32x4 kpre[NLD], vpre[NLD];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / CPR, c = idx % CPR;
            const int key = kt * BN + r;
            if (key < N) {
                kpre[i] = ld16(Kh + size_t(key) * D + 8 * c);
                vpre[i] = ld16(Vh + size_t(key) * D + 8 * c);
            } else {
                kpre[i] = u32x4{0, 0, 0, 0};
                vpre[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int stage) {
        bf16* Ks = smem + stage * 2 * TILE;
        bf16* Vs = Ks + TILE;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / CPR, c = idx % CPR;
            st16(Ks + r * D + 8 * swz_row<D>(r, c), kpre[i]);
            st16(Vs + r * D + 8 * swz_tr<D>(r, c), vpre[i]);
        }
    };

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -INFINITY;  // running max, in log2 units of the scaled scores
    float l = 0.f;        // running sum of this lane's keys (halves merged at the end)

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const int stage = kt & 1;
        if (kt + 1 < ntiles) gload(kt + 1);
        const bf16* Ks = smem + stage * 2 * TILE;
        const bf16* Vs = Ks + TILE;
        const int kstart = kt * BN;

        if (!CAUSAL || kstart <= wq0 + 31) {
            // S^T blocks: s[kb][r] = score(key = kstart + 32kb + 8(r/4) + 4hi + r%4, query = qrow)
            f32x16 s[BN / 32];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                s[kb] = f32x16{};
#pragma unroll
                for (int c = 0; c < D / 16; ++c) {
                    const bf16x8 a = as_bf16x8(ld16(Ks + off_row<D>(kb * 32 + l32, 16 * c + 8 * hi)));
                    s[kb] = mfma_32x32x16(a, qreg[c], s[kb]);
                }
            }
            const bool need_mask = (CAUSAL && kstart + BN - 1 > wq0) || (kstart + BN > N);
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float t = s[kb][r] * p.scale_log2;
                    if (need_mask) {
                        const int key = kstart + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        if ((CAUSAL && key > qrow) || key >= N) t = -INFINITY;
                    }
                    s[kb][r] = t;
                    mx = fmaxf(mx, t);
                }
            }
            mx = half_swap_max(mx);
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            m = m_new;
            float rs = 0.f;
            bf16x8 pb[BN / 32][2];
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(s[kb][r] - m_new);
                    s[kb][r] = e;
                    rs += e;
                }
                pb[kb][0] = to_bf16x8(s[kb][0], s[kb][1], s[kb][2], s[kb][3], s[kb][4], s[kb][5], s[kb][6], s[kb][7]);
                pb[kb][1] = to_bf16x8(s[kb][8], s[kb][9], s[kb][10], s[kb][11], s[kb][12], s[kb][13], s[kb][14],
                                      s[kb][15]);
            }
            l = l * alpha + rs;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            // O^T += V^T P^T.  Contraction slot (cc, hi, sl) <-> key 32kb + 16cc + 8(sl/4) + 4hi + sl%4.
            const int trow = 4 * hi + ((lane & 15) >> 2);
            const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
                    for (int cc = 0; cc < 2; ++cc) {
                        const int key = kb * 32 + 16 * cc + trow;
                        const bf16x4 v0 = lds_read_tr(Vs + off_tr<D>(key, db * 32 + tcol));
                        const bf16x4 v1 = lds_read_tr(Vs + off_tr<D>(key + 8, db * 32 + tcol));
                        o[db] = mfma_32x32x16(cat(v0, v1), pb[kb][cc], o[db]);
                    }
                }
            }
        }
        if (kt + 1 < ntiles) lstore(stage ^ 1);
        __syncthreads();
    }

    // Epilogue: O = acc / l (bf16, round to nearest even), LSE = ln2 (m + log2 l).
    const float lt = half_swap_sum(l);
    const float inv = 1.f / lt;
    if (qrow < N) {
        bf16* orow = Oh + size_t(qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x4 v = bf16x4{(bf16)(o[db][4 * j + 0] * inv), (bf16)(o[db][4 * j + 1] * inv),
                                        (bf16)(o[db][4 * j + 2] * inv), (bf16)(o[db][4 * j + 3] * inv)};
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * j + 4 * hi) = v;
            }
        }
        if (hi == 0 && p.LSE != nullptr) p.LSE[size_t(b * p.Hq + h) * N + qrow] = (m + fast_log2(lt)) * kLn2;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_bf16_t(FwdParams p, hipStream_t stream) {
    auto kern = fwd_bf16_kernel<D, CAUSAL>;
    constexpr size_t lds = fwd_lds_bytes<D>();
    static bool attr_set = false;  // benign race: setting it twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    p.nqb = (p.N + kBM - 1) / kBM;
    const long long blocks = (long long)p.nqb * p.B * p.Hq;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(256), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(FwdParams p, int d, int causal, hipStream_t stream) {
    switch (d) {
        case 64: return causal ? launch_fwd_bf16_t<64, true>(p, stream) : launch_fwd_bf16_t<64, false>(p, stream);
        case 128: return causal ? launch_fwd_bf16_t<128, true>(p, stream) : launch_fwd_bf16_t<128, false>(p, stream);
        case 256: return causal ? launch_fwd_bf16_t<256, true>(p, stream) : launch_fwd_bf16_t<256, false>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
