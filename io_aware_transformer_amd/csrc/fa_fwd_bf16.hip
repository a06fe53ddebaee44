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
// while keys/values are shared): one workgroup of NW waves per
// (batch, query head, block of BM = 32*QR*NW query rows); each wave owns
// QR blocks of 32 query rows; K/V tiles of BN keys are copied global->LDS
// by the direct-to-LDS load path (no VGPR staging), multi-buffered, and
// read by every wave.  With QR = 2 every K/V fragment read from LDS feeds two
// matrix products, halving LDS traffic per FLOP.
//
// Per wave, row block and 32-key block, in the layouts of fa_device.hpp:
//   S^T (32 keys x 32 queries) = K_blk . Q^T     A = K rows (LDS), B = Q (regs)
//   lane l then holds one query (l % 32) and 16 of its keys, so the row
//   max/sum are in-lane plus one v_permlane32_swap across the halves.
//   O^T (d x 32 queries) += V^T . P^T            A = V^T via ds_read_b64_tr_b16,
//   B = P^T straight from the score registers (the key order inside the
//   contraction is permuted consistently on both operands).
// Scores are scaled by c = |scale|*log2(e) so the exponentials are exp2
// (v_exp_f32) and p = exp2(c*s - m) is one FMA; LSE is converted back to a
// natural log at the end.  A negative scale is handled by negating Q (exact
// in bf16), a zero scale by zeroing Q, so the kernel only sees c > 0.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <math.h>

namespace fa {

namespace {

// Tile configuration per head dim: waves per workgroup (each wave owns 32
// query rows), keys per tile, LDS stages, waves per SIMD the register
// budget is cut for.
template <int D>
struct FwdCfg;
#ifndef FA_FWD_BN128
#define FA_FWD_BN128 64
#endif
#ifndef FA_FWD_BN64
#define FA_FWD_BN64 64
#endif
#ifndef FA_FWD_NW
#define FA_FWD_NW 4
#endif
template <int NW_, int BN_, int NST_, int WPE_>
struct FwdCfgT {
    static constexpr int NW = NW_, BN = BN_, NST = NST_, WPE = WPE_;
};
template <>
struct FwdCfg<64> : FwdCfgT<FA_FWD_NW, FA_FWD_BN64, 2, 2> {};
template <>
struct FwdCfg<128> : FwdCfgT<FA_FWD_NW, FA_FWD_BN128, 2, 2> {};
template <>
struct FwdCfg<256> : FwdCfgT<4, 32, 2, 1> {};

// Rescale threshold in log2 units.  0: the running max follows the row max
// exactly (the recurrence as stated; factors of exactly 1 are skipped).
// > 0: the reference max is only moved when the row max exceeds it by more
// than kTau, so exponentials stay <= 2^kTau: O = sum_j e_j v_j / sum_j e_j
// and LSE = m + log2(sum_j e_j) are the same quantities for any reference m,
// and bf16 P keeps its relative precision at any magnitude.  With 4 the
// O / l rescale (64 multiplies per lane at d = 128) runs on few tiles
// instead of nearly every one; exponentials stay <= 16, the row sum <= 16 N.
// Larger thresholds leave a sharp row's dominant term at 2^delta, rounded to
// bf16, instead of exactly 1 more often: at 8 the O error of sharp softmaxes
// grows measurably, at 4 it does not.
#ifndef FA_FWD_TAU
#define FA_FWD_TAU 4.0f
#endif
constexpr float kTau = FA_FWD_TAU;

// 1: d = 64 / 128 use the ping-pong kernel below; 0: the single-group kernel.
#ifndef FA_FWD_PP
#define FA_FWD_PP 1
#endif

template <int D>
constexpr int fwd_bm() {
    return 32 * FwdCfg<D>::NW;
}
template <int D>
constexpr size_t fwd_lds_bytes() {
    return size_t(FwdCfg<D>::NST) * 2 /*K,V*/ * FwdCfg<D>::BN * D * sizeof(bf16);
}

// Workgroup id -> (query block, batch, head).  Heaviest causal query blocks
// are issued first; units are ordered over the XCDs by order_unit.
__device__ __forceinline__ void fwd_decompose(int id, int units, int nqb, int Hq, bool causal, bool packed, int& qb,
                                              int& b, int& h) {
    const int slot = id / units;
    const int u = id - slot * units;
    qb = causal ? nqb - 1 - slot : slot;
    const int unit = order_unit(u, units, Hq, packed);
    b = unit / Hq;
    h = unit - b * Hq;
}

// K/V tiles are copied global -> LDS by the direct-to-LDS load path (no
// VGPR staging) in 1 KB pieces, one per wave instruction: lane l of piece p
// writes 16-byte slot 64p + l and fetches the chunk that the tile's slab
// layout (K slabs / V slabs, fa_device.hpp) places in that slot.  Each copy
// goes through a buffer resource whose base is the first row of the tile,
// so a lane's byte offset is the same for every tile.  On the tail tile,
// rows at or past N are clamped to row N-1 (read in bounds, masked later).
template <int D, int BN, int NW>
struct TileCopy {
    static constexpr int PIECES = BN * D * 2 / 1024;
    static constexpr int PER_WAVE = PIECES / NW;
    static_assert(PIECES % NW == 0, "tile pieces must split evenly over the waves");
    // In-tile byte offset (2 * (row * D + first element)) of each piece this lane copies.
    uint32_t koff[PER_WAVE], voff[PER_WAVE];
    int piece0;  // first piece of this wave (uniform)

    __device__ __forceinline__ void init(int w, int lane) {
        piece0 = w;
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int s = (w + NW * i) * 64 + lane;
            int r, e0;
            kslab_slot<BN>(s, r, e0);
            koff[i] = uint32_t(2 * (r * D + e0));
            vslab_slot<BN>(s, r, e0);
            voff[i] = uint32_t(2 * (r * D + e0));
        }
    }
    __device__ __forceinline__ void issue(const bf16* Kh, const bf16* Vh, bf16* Ks, bf16* Vs, int key0, int N) const {
        const uint32_t bytes = uint32_t(N - key0) * uint32_t(D * 2);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kh + size_t(key0) * D, bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vh + size_t(key0) * D, bytes);
        if (key0 + BN <= N) {
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const int piece = piece0 + NW * i;
                buf16_to_lds(kr, koff[i], Ks + piece * 512);
                buf16_to_lds(vr, voff[i], Vs + piece * 512);
            }
        } else {
            const uint32_t last = uint32_t(N - 1 - key0);  // last valid row of the tile
#pragma unroll
            for (int i = 0; i < PER_WAVE; ++i) {
                const int piece = piece0 + NW * i;
                const uint32_t rk = koff[i] / (2 * D), rv = voff[i] / (2 * D);
                const uint32_t ok = min(rk, last) * (2 * D) + koff[i] % (2 * D);
                const uint32_t ov = min(rv, last) * (2 * D) + voff[i] % (2 * D);
                buf16_to_lds(kr, ok, Ks + piece * 512);
                buf16_to_lds(vr, ov, Vs + piece * 512);
            }
        }
    }
};

template <int D, int MASK>
__global__ __launch_bounds__(FwdCfg<D>::NW * 64) __attribute__((amdgpu_waves_per_eu(FwdCfg<D>::WPE, FwdCfg<D>::WPE)))
void fwd_bf16_kernel(FwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK == 2;  // left bound in use (every wl_ test is guarded by it)
    const int wl_ = MASK == 2 ? p.wl : kUnbounded;
    const int wr_ = MASK == 2 ? p.wr : 0;
    constexpr int NW = FwdCfg<D>::NW, BN = FwdCfg<D>::BN, NST = FwdCfg<D>::NST;
    constexpr int BM = 32 * NW;
    constexpr int TILE = BN * D;
    constexpr int KB = BN / 32;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;  // > 0

    int qb, b, h;
    fwd_decompose(blockIdx.x, p.B * p.Hq, p.nqb, p.Hq, CAUSAL, p.cu != nullptr, qb, b, h);
    const int g = h / (p.Hq / p.Hkv);
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    if (qb * BM >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const size_t qoff = sq.qrow(h) * D;
    const size_t kvoff = sq.kvrow(g) * D;
    const bf16* __restrict__ Qh = static_cast<const bf16*>(p.Q) + qoff;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;
    bf16* __restrict__ Oh = static_cast<bf16*>(p.O) + qoff;

    const int q0 = qb * BM;
    const int wq0 = q0 + 32 * w;  // first query row of this wave (uniform)
    const int wq_last = wq0 + 31;
    const int qrow = wq0 + l32;   // the query row of this lane

    // Key tiles [kt0, kt0 + ntiles); masked kernels see keys q - wl .. q + wr.
    const int kend = CAUSAL ? min(N, q0 + BM + wr_) : N;
    const int kt0 = WIN ? max(0, q0 - wl_) / BN : 0;
    const int ntiles = (kend + BN - 1) / BN - kt0;

    TileCopy<D, BN, NW> cp;
    cp.init(w, lane);
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
        if (st < ntiles) cp.issue(Kh, Vh, smem + st * 2 * TILE, smem + st * 2 * TILE + TILE, (kt0 + st) * BN, N);

    // Q rows of this wave as MFMA B operands: Q[qrow][16cc + 8hi .. +7].
    // qmode 1 negates (negative scale), 2 zeroes (zero scale).
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (qrow < N && p.qmode != 2) v = ld16(Qh + size_t(qrow) * D + 16 * cc + 8 * hi);
        if (p.qmode == 1) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qreg[cc] = as_bf16x8(v);
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    float m = -3.0e38f;  // running (reference) max of c*s; finite floor (rows masked in early tiles)
    float l = 0.f;        // running sum over this lane's keys (halves merged at the end)
    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    // Row limit for masking: keys above it are hidden (causal and/or past N).
    const int key_lim = CAUSAL ? min(qrow + wr_, N - 1) : N - 1;
    const int key_lo = WIN ? qrow - wl_ : 0;

    wait_vmem();
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        {
            const int nt = kt + NST - 1;
            if (nt < ntiles) {
                bf16* st = smem + (nt % NST) * 2 * TILE;
                cp.issue(Kh, Vh, st, st + TILE, (kt0 + nt) * BN, N);
            }
        }
        const bf16* Ks = smem + (kt % NST) * 2 * TILE;
        const bf16* Vs = Ks + TILE;
        const int kstart = (kt0 + kt) * BN;

        if (!CAUSAL || (kstart <= wq_last + wr_ && (!WIN || kstart + BN - 1 >= wq0 - wl_))) {
            // S^T blocks: s[kb][r] = score(key kstart + 32kb + 8(r/4) + 4hi + r%4, query qrow).
            // The KB accumulation chains are interleaved so consecutive MFMAs are independent.
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    if (CAUSAL && kstart + 32 * kb > wq_last + wr_) continue;
                    const bf16x8 a = as_bf16x8(ld16(Ks + kslab_off<BN>(kb * 32 + l32, 16 * cc + 8 * hi)));
                    s[kb] = mfma_32x32x16(a, qreg[cc], s[kb]);
                }
            }
            const bool need_mask =
                (CAUSAL && (kstart + BN - 1 > wq0 + wr_ || (WIN && kstart < wq_last - wl_))) || (kstart + BN > N);
            if (need_mask) {
                const int lim = key_lim - kstart - 4 * hi;
                const int lo = key_lo - kstart - 4 * hi;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = kb * 32 + 8 * (r >> 2) + (r & 3);
                        s[kb][r] = (kk > lim || (WIN && kk < lo)) ? -INFINITY : s[kb][r];
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = half_swap_max(mx) * c;
            // Rescale only when some row of this wave raised its max (by more
            // than kTau): otherwise every factor exp(m_old - m_new) is exactly
            // 1 and the multiply is skipped.  The branch is wave-uniform.
            if (__any(mx > m + kTau)) {
                const float m_new = fmaxf(m, mx);
                const float alpha = fast_exp2(m - m_new);
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
            }
            bf16x8 pb[KB][2];
            float rs = 0.f;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = fast_exp2(fmaf(s[kb][r], c, -m));
                    s[kb][r] = e;
                    rs += e;
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    pb[kb][cc] = to_bf16x8(s[kb][8 * cc + 0], s[kb][8 * cc + 1], s[kb][8 * cc + 2], s[kb][8 * cc + 3],
                                           s[kb][8 * cc + 4], s[kb][8 * cc + 5], s[kb][8 * cc + 6], s[kb][8 * cc + 7]);
            }
            l += rs;
            // O^T += V^T P^T.  Contraction slot (cc, hi, sl) <-> key 32kb + 16cc + 8(sl/4) + 4hi + sl%4.
            // Consecutive MFMAs update different dim blocks (independent accumulators).
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if (CAUSAL && kstart + 32 * kb > wq_last + wr_) continue;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int key = kb * 32 + 16 * cc + trow;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const bf16x4 v0 = lds_read_tr(Vs + vslab_off<BN>(key, db * 32 + tcol));
                        const bf16x4 v1 = lds_read_tr(Vs + vslab_off<BN>(key + 8, db * 32 + tcol));
                        o[db] = mfma_32x32x16(cat(v0, v1), pb[kb][cc], o[db]);
                    }
                }
            }
        }
        wait_vmem();
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
        if (hi == 0 && p.LSE != nullptr) p.LSE[sq.qrow(h) + qrow] = (m + fast_log2(lt)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Ping-pong forward (d = 64, 128).  Two waves share every SIMD; if both ran
// the same phase (matrix products, then softmax) at the same time, the
// matrix cores would idle during the softmax.  Here the 8 waves of a
// workgroup form two groups of 4 (one wave of each group per SIMD) that run
// the same software pipeline one phase apart:
//   M phase j:  O^T += V_{j-1}^T P_{j-1}^T   and   S_j^T = K_j Q^T   (MFMA)
//   V phase j:  softmax of S_j (max, rescale, exp2, sum, bf16 P_j)   (VALU)
// While group A is in an M phase, group B is in a V phase and vice versa;
// a workgroup barrier closes every phase and keeps the offset.  K/V tiles
// are triple-buffered in LDS: tile j is read from A's M phase j to B's M
// phase j+1, and tile j+3 is copied into its buffer two phases before it is
// first needed.  Group A owns query rows q0 .. q0+127, group B q0+128 ..
// q0+255.
// ---------------------------------------------------------------------------
template <int D>
struct PPCfg;
template <>
struct PPCfg<64> {
    static constexpr int BN = FA_FWD_BN64;
};
template <>
struct PPCfg<128> {
    static constexpr int BN = FA_FWD_BN128;
};
constexpr int kPPWaves = 8;
constexpr int kPPStages = 3;
constexpr int kPPBM = 32 * kPPWaves;

template <int D>
constexpr size_t pp_lds_bytes() {
    // K/V stages plus two V^T buffers
    return (size_t(kPPStages) * 2 + 2) * PPCfg<D>::BN * D * sizeof(bf16);
}

// V^T tile layout: element (dim, key) of a D x BN tile.  Keys are grouped
// by 16; inside a group the order is [4hi+0..3, 8+4hi+0..3] for hi = 0, 1,
// which is the key order of the MFMA A operand, so one 16-byte read gives a
// lane its 8 keys; the two 16-byte halves of a row are swapped when bit 3
// of the dim is set (conflict-free reads of 16 consecutive dims).
template <int D>
__device__ __forceinline__ int vt_off(int dim, int key) {
    return (key >> 4) * D * 16 + dim * 16 + 8 * (((key >> 2) & 1) ^ ((dim >> 3) & 1)) + 4 * ((key >> 3) & 1) +
           (key & 3);
}

template <int D, int MASK>
__global__ __launch_bounds__(kPPWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(FwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK == 2;  // left bound in use (every wl_ test is guarded by it)
    const int wl_ = MASK == 2 ? p.wl : kUnbounded;
    const int wr_ = MASK == 2 ? p.wr : 0;
    constexpr int BN = PPCfg<D>::BN;
    constexpr int NST = kPPStages;
    constexpr int BM = kPPBM;
    constexpr int TILE = BN * D;
    constexpr int KB = BN / 32;
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int grp = w >> 2;                                  // 0: group A, 1: group B
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;  // > 0

    int qb, b, h;
    fwd_decompose(blockIdx.x, p.B * p.Hq, p.nqb, p.Hq, CAUSAL, p.cu != nullptr, qb, b, h);
    const int g = h / (p.Hq / p.Hkv);
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    if (qb * BM >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const size_t qoff = sq.qrow(h) * D;
    const size_t kvoff = sq.kvrow(g) * D;
    const bf16* __restrict__ Qh = static_cast<const bf16*>(p.Q) + qoff;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;
    bf16* __restrict__ Oh = static_cast<bf16*>(p.O) + qoff;

    const int q0 = qb * BM;
    const int wq0 = q0 + 32 * w;  // first query row of this wave (uniform)
    const int wq_last = wq0 + 31;
    const int qrow = wq0 + l32;

    // Key tiles of the workgroup: [kt0, kt0 + T).  Masked kernels see keys
    // q - wl .. q + wr of each query q (causal: wl unbounded, wr = 0).
    const int kend = CAUSAL ? min(N, q0 + BM + wr_) : N;
    const int kt0 = WIN ? max(0, q0 - wl_) / BN : 0;
    const int T = (kend + BN - 1) / BN - kt0;

    TileCopy<D, BN, kPPWaves> cp;
    cp.init(w, lane);
#pragma unroll
    for (int t = 0; t < NST; ++t)
        if (t < T) cp.issue(Kh, Vh, smem + t * 2 * TILE, smem + t * 2 * TILE + TILE, (kt0 + t) * BN, N);

    bf16x8 qreg[D / 16];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (qrow < N && p.qmode != 2) v = ld16(Qh + size_t(qrow) * D + 16 * cc + 8 * hi);
        if (p.qmode == 1) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qreg[cc] = as_bf16x8(v);
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    f32x16 s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x16{};
    bf16x8 pb[KB][2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) pb[kb][0] = pb[kb][1] = bf16x8{};
    // Finite floor for the running max: a row whose first tiles are all
    // masked (left window edge) keeps exp2(m_old - m_new) defined.
    float m = -3.0e38f, l = 0.f;
    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int key_lim = CAUSAL ? min(qrow + wr_, N - 1) : N - 1;  // last visible key of this row
    const int key_lo = WIN ? qrow - wl_ : 0;                     // first visible key

    // Number of 32-key blocks of tile j this wave must process (uniform).
    auto active_kb = [&](int j) -> int {
        if (!CAUSAL) return KB;
        const int kstart = (kt0 + j) * BN;
        if (kstart > wq_last + wr_ || (WIN && kstart + BN - 1 < wq0 - wl_)) return 0;
        return min(KB, (wq_last + wr_ - kstart) / 32 + 1);
    };

    wait_vmem();
    __syncthreads();

    // Per-lane element offset of the V^T A-operand read (dim l32 of a 32-dim
    // block, the 8 keys of half hi of a 16-key group).
    const int vt_lane = vt_off<D>(l32, 4 * hi);
    // Transpose tile j's V (V slabs) into V^T buffer j % 2.  Done by the 4
    // waves of group A in their V phase; each transposing read returns 4
    // consecutive keys of one dim, written back as one 8-byte store.
    constexpr int TR_PER_WAVE = (BN / 8) * (D / 32) / 4;
    auto transpose_v = [&](int j, bf16x4 (&buf)[TR_PER_WAVE], bool write) {
        const bf16* Vs = smem + (j % NST) * 2 * TILE + TILE;
        bf16* VT = smem + (2 * NST + (j & 1)) * TILE;
#pragma unroll
        for (int i = 0; i < TR_PER_WAVE; ++i) {
            const int t = w + 4 * i;  // instruction index 0 .. (BN/8)(D/32) - 1
            const int kb8 = t / (D / 32), db = t - (t / (D / 32)) * (D / 32);
            if (!write) {
                buf[i] = lds_read_tr(Vs + vslab_off<BN>(8 * kb8 + trow, db * 32 + tcol));
            } else {
                *reinterpret_cast<bf16x4*>(VT + vt_off<D>(db * 32 + l32, 8 * kb8 + 4 * hi)) = buf[i];
            }
        }
    };

    // Steps 0 .. 2T+1, one workgroup barrier after each.  Group A: step 2j is
    // its M phase j, step 2j+1 its V phase j.  Group B runs one step later.
    // K/V refill: at even step 2t-2 (t >= 3) tile t goes into the buffer of
    // tile t-3, whose last reader (group B, M phase t-2) finished in the
    // previous step; the copy is waited for at the end of the next (odd) step.
    auto refill = [&](int step) {
        if (!(step & 1) && step >= 4) {
            const int t = step / 2 + 1;
            if (t < T) {
                bf16* st = smem + (t % NST) * 2 * TILE;
                cp.issue(Kh, Vh, st, st + TILE, (kt0 + t) * BN, N);
            }
        }
    };
    auto finish = [&](int step) {
        if ((step & 1) && step >= 5) wait_vmem();
        wait_lds();  // this wave's LDS writes are done
        __builtin_amdgcn_s_barrier();
    };
    // ---- M phase j: PV of tile j-1, then QK of tile j.  LDS fragments are
    // loaded one block ahead of the MFMAs that use them; scheduling barriers
    // keep at most two blocks live.
    auto phase_m = [&](int j) {
        if (j >= 1 && active_kb(j - 1) > 0) {
            // V^T of tile j-1 (written by group A in its V phase j-1): one
            // 16-byte read per A operand.
            const bf16* VT = smem + (2 * NST + ((j - 1) & 1)) * TILE + vt_lane;
            bf16x8 fa[D / 32], fb[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) fa[db] = as_bf16x8(ld16(VT + db * 32 * 16));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db) fb[db] = as_bf16x8(ld16(VT + (2 * kb + 1) * D * 16 + db * 32 * 16));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] = mfma_32x32x16(fa[db], pb[kb][0], o[db]);
                __builtin_amdgcn_sched_barrier(0);
                if (kb + 1 < KB) {
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        fa[db] = as_bf16x8(ld16(VT + (2 * kb + 2) * D * 16 + db * 32 * 16));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] = mfma_32x32x16(fb[db], pb[kb][1], o[db]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (j < T && active_kb(j) > 0) {
            const bf16* Ks = smem + (j % NST) * 2 * TILE;
            bf16x8 ka[KB], kbf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = f32x16{};
                ka[kb] = as_bf16x8(ld16(Ks + kslab_off<BN>(kb * 32 + l32, 8 * hi)));
            }
#pragma unroll
            for (int cc = 0; cc < D / 16; cc += 2) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    kbf[kb] = as_bf16x8(ld16(Ks + kslab_off<BN>(kb * 32 + l32, 16 * (cc + 1) + 8 * hi)));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[kb] = mfma_32x32x16(ka[kb], qreg[cc], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
                if (cc + 2 < D / 16) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        ka[kb] = as_bf16x8(ld16(Ks + kslab_off<BN>(kb * 32 + l32, 16 * (cc + 2) + 8 * hi)));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[kb] = mfma_32x32x16(kbf[kb], qreg[cc + 1], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // ---- V phase j: online softmax of S_j -> P_j (bf16), O rescaled if needed.
    auto phase_v = [&](int j) {
        if (j >= T || active_kb(j) == 0) return;
        const int kstart = (kt0 + j) * BN;
        const bool mask_hi = (CAUSAL && kstart + BN - 1 > wq0 + wr_) || (kstart + BN > N);
        const bool mask_lo = WIN && kstart < wq_last - wl_;
        if (mask_hi && !mask_lo) {
            const int lim = key_lim - kstart - 4 * hi;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) ? -INFINITY : s[kb][r];
        } else if (mask_lo) {
            const int lim = key_lim - kstart - 4 * hi;
            const int lo = key_lo - kstart - 4 * hi;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = kb * 32 + 8 * (r >> 2) + (r & 3);
                    s[kb][r] = (kk > lim || kk < lo) ? -INFINITY : s[kb][r];
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = half_swap_max(mx) * c;
        if (__any(mx > m + kTau)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            m = m_new;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        }
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float e[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                e[r] = fast_exp2(fmaf(s[kb][r], c, -m));
                rs += e[r];
            }
            pb[kb][0] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
            pb[kb][1] = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
        }
        l += rs;
    };

    if (grp == 0) {
        for (int j = 0; j <= T; ++j) {
            refill(2 * j);
            phase_m(j);
            finish(2 * j);
            refill(2 * j + 1);
            if (j < T) {
                bf16x4 tb[TR_PER_WAVE];
                transpose_v(j, tb, false);
                phase_v(j);
                transpose_v(j, tb, true);
            }
            finish(2 * j + 1);
        }
    } else {
        finish(0);
        for (int j = 0; j <= T; ++j) {
            refill(2 * j + 1);
            phase_m(j);
            finish(2 * j + 1);
            if (j < T) {
                refill(2 * j + 2);
                phase_v(j);
                finish(2 * j + 2);
            }
        }
    }

    const float lt = half_swap_sum(l);
    const float inv = 1.f / lt;
    if (qrow < N) {
        bf16* orow = Oh + size_t(qrow) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const bf16x4 v = bf16x4{(bf16)(o[db][4 * jj + 0] * inv), (bf16)(o[db][4 * jj + 1] * inv),
                                        (bf16)(o[db][4 * jj + 2] * inv), (bf16)(o[db][4 * jj + 3] * inv)};
                *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * jj + 4 * hi) = v;
            }
        }
        if (hi == 0 && p.LSE != nullptr) p.LSE[sq.qrow(h) + qrow] = (m + fast_log2(lt)) * kLn2;
    }
}

template <int D, int MASK>
hipError_t launch_fwd_pp_t(FwdParams p, hipStream_t stream) {
    auto kern = fwd_pp_kernel<D, MASK>;
    constexpr size_t lds = pp_lds_bytes<D>();
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    p.nqb = (p.N + kPPBM - 1) / kPPBM;
    const long long blocks = (long long)p.nqb * p.B * p.Hq;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kPPWaves * 64), lds, stream, p);
    return hipGetLastError();
}

template <int D, int MASK>
hipError_t launch_fwd_bf16_t(FwdParams p, hipStream_t stream) {
    auto kern = fwd_bf16_kernel<D, MASK>;
    constexpr size_t lds = fwd_lds_bytes<D>();
    static bool attr_set = false;  // benign race: setting it twice is harmless
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    constexpr int BM = fwd_bm<D>();
    p.nqb = (p.N + BM - 1) / BM;
    const long long blocks = (long long)p.nqb * p.B * p.Hq;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(FwdCfg<D>::NW * 64), lds, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(FwdParams p, int d, int causal, hipStream_t stream) {
    // Only c = scale*log2(e) > 0 reaches the kernel (see the header comment).
    if (p.scale_log2 > 0.f) {
        p.qmode = 0;
    } else if (p.scale_log2 < 0.f) {
        p.qmode = 1;
        p.scale_log2 = -p.scale_log2;
    } else {
        p.qmode = 2;
        p.scale_log2 = 1.f;
    }
    // 0: no mask, 1: causal, 2: a general window
    const int mk = !causal ? 0 : (p.wl >= kUnbounded && p.wr == 0) ? 1 : 2;
#define FA_FWD_DISPATCH(L, DD) \
    (mk == 0 ? L<DD, 0>(p, stream) : mk == 1 ? L<DD, 1>(p, stream) : L<DD, 2>(p, stream))
    switch (d) {
#if FA_FWD_PP
        case 64: return FA_FWD_DISPATCH(launch_fwd_pp_t, 64);
        case 128: return FA_FWD_DISPATCH(launch_fwd_pp_t, 128);
#else
        case 64: return FA_FWD_DISPATCH(launch_fwd_bf16_t, 64);
        case 128: return FA_FWD_DISPATCH(launch_fwd_bf16_t, 128);
#endif
        case 256: return FA_FWD_DISPATCH(launch_fwd_bf16_t, 256);
        default: return hipErrorInvalidValue;
    }
#undef FA_FWD_DISPATCH
}

}  // namespace fa
