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
// while keys/values are shared): one workgroup of 8 waves per
// (batch, query head, block of 256 query rows); each wave owns 32 query
// rows; K/V tiles of BN keys are copied global->LDS by the direct-to-LDS
// load path (no VGPR staging) through four stages and read by every wave.
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
constexpr float kTau = 4.0f;

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

// ---------------------------------------------------------------------------
// Ping-pong forward (d = 64, 128, 256).  Two waves share every SIMD; if both ran
// the same phase (matrix products, then softmax) at the same time, the
// matrix cores would idle during the softmax.  Here the 8 waves of a
// workgroup form two groups of 4 (one wave of each group per SIMD) that run
// the same software pipeline one phase apart:
//   M phase j:  O^T += V_{j-1}^T P_{j-1}^T   and   S_j^T = K_j Q^T   (MFMA)
//   V phase j:  softmax of S_j (max, rescale, exp2, sum, bf16 P_j)   (VALU)
// While group A is in an M phase, group B is in a V phase and vice versa;
// a workgroup barrier closes every phase and keeps the offset.  The V^T
// operand of O^T += V^T P^T is read straight from the row-major V tile with
// transposing LDS reads (ds_read_b64_tr_b16), so both groups' V phases are
// the softmax alone.  K/V tiles go through four LDS stages: tile t is read
// from A's M phase t to B's M phase t+1, and is copied into the stage of
// tile t-4 at step 2t-4, four phases before its first use; each wave waits
// only for its own copies of the tile about to be read (the newer tile may
// stay in flight).  Group A owns query rows q0 .. q0+127, group B
// q0+128 .. q0+255.
// ---------------------------------------------------------------------------
constexpr int kPPWaves = 8;
constexpr int kPPStages = 4;
constexpr int kPPBM = 32 * kPPWaves;

// Keys per tile: 64, or 32 at d = 256 so that four K/V stages fit in LDS
// (128 KB) and a wave's registers hold O (128), Q (64) and one S block.
template <int D>
constexpr int pp_bn() {
    return D == 256 ? 32 : 64;
}
template <int D>
constexpr size_t pp_lds_bytes() {
    return size_t(kPPStages) * 2 * pp_bn<D>() * D * sizeof(bf16);
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time: the
// count is an immediate, so dispatch over the values the kernel uses.
template <int STEP>
__device__ __forceinline__ void wait_vmem_at_most(int n_groups) {
    switch (n_groups) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F70 | (1 * STEP)); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * STEP)); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70 | (3 * STEP)); break;
    }
}

template <int D, int MASK, bool DROP>
__global__ __launch_bounds__(kPPWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(FwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr); 3: the block map p.bmask together
    // with the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK >= 2;  // left bound in use (every wl_ test is guarded by it)
    constexpr bool SPARSE = MASK == 3;
    const int wl_ = MASK >= 2 ? p.wl : kUnbounded;
    const int wr_ = MASK >= 2 ? p.wr : 0;
    constexpr int BN = pp_bn<D>();
    constexpr int NST = kPPStages;
    constexpr int BM = kPPBM;
    constexpr int TILE = BN * D;
    constexpr int KB = BN / 32;
    using Copy = TileCopy<D, BN, kPPWaves>;
    constexpr int CPW = 2 * Copy::PER_WAVE;  // copy instructions per wave per tile
    static_assert(CPW * 3 < 16, "vmcnt immediates stay in the low field");
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
    int T = (kend + BN - 1) / BN - kt0;
    // Block-sparse: the tiles of that range whose map block is visible to
    // group A (map row q0 / 128, tag bit 0) or group B (the next row, bit 1),
    // listed in LDS after the stages; j below then indexes the list.
    int* const tlist = reinterpret_cast<int*>(smem_raw + pp_lds_bytes<D>());
    if constexpr (SPARSE) {
        const int r0 = q0 / kSparseBlock;
        if (w == 0) {
            const int cnt = compact_tiles(tlist, T, lane, [&](int t) {
                const int col = (kt0 + t) * BN / kSparseBlock;
                return int(p.bmask[size_t(r0) * p.nb + col] != 0) |
                       (r0 + 1 < p.nb && p.bmask[size_t(r0 + 1) * p.nb + col] != 0 ? 2 : 0);
            });
            if (lane == 0) tlist[kSparseListCap] = cnt;
        }
        __syncthreads();
        T = __builtin_amdgcn_readfirstlane(lds_i32(tlist + kSparseListCap));
    }
    // First key of tile j, and (block-sparse) which groups see it.
    auto tile_key0 = [&](int j) -> int {
        if constexpr (SPARSE) return (kt0 + (__builtin_amdgcn_readfirstlane(lds_i32(tlist + j)) & 0xFFFFFF)) * BN;
        else return (kt0 + j) * BN;
    };
    auto group_sees = [&](int j) -> bool {
        if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(lds_i32(tlist + j)) >> (24 + grp)) & 1;
        else return true;
    };

    // Q rows first (the oldest loads of the wave), then the prologue tiles
    // 0 .. min(T, NST) - 1 into the empty stages.
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
        u32x4 v = u32x4{0, 0, 0, 0};
        if (qrow < N && p.qmode != 2) v = ld16(Qh + size_t(qrow) * D + 16 * cc + 8 * hi);
        if (p.qmode == 1) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        qreg[cc] = as_bf16x8(v);
    }
    Copy cp;
    cp.init(w, lane);
#pragma unroll
    for (int t = 0; t < NST; ++t)
        if (t < T) cp.issue(Kh, Vh, smem + t * 2 * TILE, smem + t * 2 * TILE + TILE, tile_key0(t), N);

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
    // Transposing reads of the V operand: lane (4e + i) of each 16-lane
    // group addresses key row e (+ 4hi) of a 16-key block, 4 dims at tcol.
    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int key_lim = CAUSAL ? min(qrow + wr_, N - 1) : N - 1;  // last visible key of this row
    const int key_lo = WIN ? qrow - wl_ : 0;                     // first visible key

    // Number of 32-key blocks of tile j this wave must process (uniform).
    auto active_kb = [&](int j) -> int {
        if (!CAUSAL) return KB;
        if (!group_sees(j)) return 0;
        const int kstart = tile_key0(j);
        if (kstart > wq_last + wr_ || (WIN && kstart + BN - 1 < wq0 - wl_)) return 0;
        return min(KB, (wq_last + wr_ - kstart) / 32 + 1);
    };

    // Tile 0 must be in LDS before step 0: wait for it (the newer prologue
    // tiles may stay in flight), then publish.
    wait_vmem_at_most<CPW>(min(T, NST) - 1);
    __syncthreads();

    // Steps 0 .. 2T+1, one workgroup barrier after each.  Group A: step 2j is
    // its M phase j, step 2j+1 its V phase j.  Group B runs one step later.
    // Refill: at even step 2u (u >= 2) tile u + 2 goes into the stage of
    // tile u - 2, whose last reader (group B, M phase u - 1: the V operand
    // of tile u - 2) finished at the previous barrier.
    auto refill = [&](int step) {
        if (!(step & 1) && step >= 4) {
            const int t = step / 2 + 2;
            if (t < T) {
                bf16* st = smem + (t % NST) * 2 * TILE;
                cp.issue(Kh, Vh, st, st + TILE, tile_key0(t), N);
            }
        }
    };
    // End of a step: before step 2t (group A reads K_t) every wave has
    // waited for its own copies of tile t.  At the end of step 2t - 1 the
    // tiles issued so far are 0 .. max(NST - 1, t + 1) (bounded by T - 1).
    auto finish = [&](int step) {
        if (step & 1) {
            const int t = (step + 1) / 2;
            if (t < T) wait_vmem_at_most<CPW>(min(T - 1, max(NST - 1, t + 1)) - t);
        }
        wait_lds();  // this wave's LDS reads are done before the stage can be refilled
        __builtin_amdgcn_s_barrier();
    };
    // ---- M phase j: PV of tile j-1, then QK of tile j.  LDS fragments are
    // loaded one block ahead of the MFMAs that use them; scheduling barriers
    // keep at most two blocks live.
    auto phase_m = [&](int j) {
        if (j >= 1 && active_kb(j - 1) > 0) {
            // V^T A operand of contraction block (kb, cc): keys
            // 32kb + 16cc + 8(sl/4) + 4hi + sl%4 of dims db*32 + l32, read
            // transposed from the V slabs of tile j-1.
            const bf16* Vs = smem + ((j - 1) % NST) * 2 * TILE + TILE;
            // Chunks of VC output dim blocks, in the order (kb, cc, chunk);
            // chunk x + 1 is loaded while the MFMAs of chunk x run.
            constexpr int VC = D / 32 > 4 ? 1 : D / 32;
            constexpr int NCH = D / 32 / VC;
            constexpr int X = KB * 2 * NCH;
            bf16x8 fv[2][VC];
            auto load_v = [&](bf16x8(&f)[VC], int x) {
                const int kb = x / (2 * NCH), cc = (x / NCH) & 1, ch = x % NCH;
                const int key = kb * 32 + 16 * cc + trow;
#pragma unroll
                for (int i = 0; i < VC; ++i) {
                    const int db = ch * VC + i;
                    const bf16x4 v0 = lds_read_tr(Vs + vslab_off<BN>(key, db * 32 + tcol));
                    const bf16x4 v1 = lds_read_tr(Vs + vslab_off<BN>(key + 8, db * 32 + tcol));
                    f[i] = cat(v0, v1);
                }
            };
            load_v(fv[0], 0);
#pragma unroll
            for (int x = 0; x < X; ++x) {
                if (x + 1 < X) load_v(fv[(x + 1) & 1], x + 1);
                __builtin_amdgcn_sched_barrier(0);
                const int kb = x / (2 * NCH), cc = (x / NCH) & 1, ch = x % NCH;
#pragma unroll
                for (int i = 0; i < VC; ++i)
                    o[ch * VC + i] = mfma_32x32x16(fv[x & 1][i], pb[kb][cc], o[ch * VC + i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (j < T && active_kb(j) > 0) {
            const bf16* Ks = smem + (j % NST) * 2 * TILE;
            bf16x8 ka[KB], kbf[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = f32x16{};
                ka[kb] = as_bf16x8(lds16(Ks + kslab_off<BN>(kb * 32 + l32, 8 * hi)));
            }
#pragma unroll
            for (int cc = 0; cc < D / 16; cc += 2) {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
                    kbf[kb] = as_bf16x8(lds16(Ks + kslab_off<BN>(kb * 32 + l32, 16 * (cc + 1) + 8 * hi)));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) s[kb] = mfma_32x32x16(ka[kb], qreg[cc], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
                if (cc + 2 < D / 16) {
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        ka[kb] = as_bf16x8(lds16(Ks + kslab_off<BN>(kb * 32 + l32, 16 * (cc + 2) + 8 * hi)));
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
        const int kstart = tile_key0(j);
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
            if constexpr (DROP) {
                // the row sum keeps every term; only P entering PV is dropped
                uint32_t y[4];
                drop_bytes_qmajor(y, qrow, kstart + 32 * kb, hi, lane, uint32_t(b * p.Hq + h), p.drop_off, p.drop_k0,
                                  p.drop_k1);
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = drop_keep(y, r, p.drop_t8) ? e[r] : 0.f;
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
            phase_v(j);
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
    // A row that sees no key at all (block-sparse only) has l = 0: O = 0,
    // LSE = -inf.  Dropout scales the kept terms by 256 / (256 - t8).
    float inv = (!SPARSE || lt > 0.f) ? 1.f / lt : 0.f;
    if constexpr (DROP) inv *= 256.f / float(256 - p.drop_t8);
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
        if (hi == 0 && p.LSE != nullptr)
            p.LSE[sq.qrow(h) + qrow] = (!SPARSE || lt > 0.f) ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
    }
}

template <int D, int MASK, bool DROP = false>
hipError_t launch_fwd_pp_t(FwdParams p, hipStream_t stream) {
    auto kern = fwd_pp_kernel<D, MASK, DROP>;
    constexpr size_t lds = pp_lds_bytes<D>() + (MASK == 3 ? size_t(kSparseListCap + 1) * sizeof(int) : 0);
    static DeviceOnce attr;
    const hipError_t e = set_max_dynamic_lds(kern, lds, attr);
    if (e != hipSuccess) return e;
    p.nqb = (p.N + kPPBM - 1) / kPPBM;
    const long long blocks = (long long)p.nqb * p.B * p.Hq;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kPPWaves * 64), lds, stream, p);
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
    // 0: no mask, 1: causal, 2: a general window, 3: block map (and window)
    const int mk = p.bmask != nullptr ? 3 : !causal ? 0 : (p.wl >= kUnbounded && p.wr == 0) ? 1 : 2;
    if (p.drop_t8 > 0) {
        // dropout: fixed-length batches, d = 64 / 128, no window (the entry point checks)
        if (d == 64) return mk == 0 ? launch_fwd_pp_t<64, 0, true>(p, stream) : launch_fwd_pp_t<64, 1, true>(p, stream);
        if (d == 128)
            return mk == 0 ? launch_fwd_pp_t<128, 0, true>(p, stream) : launch_fwd_pp_t<128, 1, true>(p, stream);
        return hipErrorNotSupported;
    }
    if (mk == 3) {
        // d = 64 / 128 only (the entry point checks)
        if (d == 64) return launch_fwd_pp_t<64, 3>(p, stream);
        if (d == 128) return launch_fwd_pp_t<128, 3>(p, stream);
        return hipErrorNotSupported;
    }
#define FA_FWD_DISPATCH(L, DD) \
    (mk == 0 ? L<DD, 0>(p, stream) : mk == 1 ? L<DD, 1>(p, stream) : L<DD, 2>(p, stream))
    switch (d) {
        case 64: return FA_FWD_DISPATCH(launch_fwd_pp_t, 64);
        case 128: return FA_FWD_DISPATCH(launch_fwd_pp_t, 128);
        case 256: return FA_FWD_DISPATCH(launch_fwd_pp_t, 256);
        default: return hipErrorInvalidValue;
    }
#undef FA_FWD_DISPATCH
}

}  // namespace fa
