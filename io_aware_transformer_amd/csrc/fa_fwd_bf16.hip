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
// q0+128 .. q0+255.  A persistent launch (STREAM) gives a workgroup several
// query blocks: their key tiles form one stream through the same stages,
// the next block's Q is loaded two steps before its first tile, and a
// block's output is written in the M phase where its last PV completes.
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

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (the
// count is an immediate; counts above 31 wait for 31, which is stricter).
__device__ __forceinline__ void wait_vmcnt(int n) {
#define FA_VMW(k) \
    case k: __builtin_amdgcn_s_waitcnt(0x0F70 | ((k) & 15) | (((k) >> 4) << 14)); break;
    switch (n) {
        FA_VMW(0) FA_VMW(1) FA_VMW(2) FA_VMW(3) FA_VMW(4) FA_VMW(5) FA_VMW(6) FA_VMW(7)
        FA_VMW(8) FA_VMW(9) FA_VMW(10) FA_VMW(11) FA_VMW(12) FA_VMW(13) FA_VMW(14) FA_VMW(15)
        FA_VMW(16) FA_VMW(17) FA_VMW(18) FA_VMW(19) FA_VMW(20) FA_VMW(21) FA_VMW(22) FA_VMW(23)
        FA_VMW(24) FA_VMW(25) FA_VMW(26) FA_VMW(27) FA_VMW(28) FA_VMW(29) FA_VMW(30)
        default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15 | (1 << 14)); break;
    }
#undef FA_VMW
}

// One (query block, batch, head) work item of the forward, as kept in the
// workgroup's item table in LDS (32 bytes).
struct PPItem {
    size_t qrow0;   // first row of the head in Q / O / LSE
    size_t kvrow0;  // first row of its key/value head in K / V
    int qb, n;      // query block, rows of the sequence
    int kt0, T;     // key tiles [kt0, kt0 + T) this block visits
};
static_assert(sizeof(PPItem) == 32, "two 16-byte LDS reads per item");
// Items one workgroup of a persistent launch takes at most.  The table is
// followed by each item's batch * H_q + head (the dropout counter) and the
// stream's total tile count.
constexpr int kPPItemCap = 512;
template <int D, int MASK>
constexpr size_t pp_table_off() {
    return pp_lds_bytes<D>() + (MASK == 3 ? size_t(kSparseListCap + 1) * sizeof(int) : 0);
}
template <int D, int MASK, bool STREAM>
constexpr size_t pp_lds_total() {
    return pp_table_off<D, MASK>() + (STREAM ? size_t(kPPItemCap) * (sizeof(PPItem) + sizeof(int)) + 16 : 0);
}

template <int D, int MASK, bool DROP, bool STREAM>
__global__ __launch_bounds__(kPPWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(FwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr); 3: the block map p.bmask together
    // with the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK >= 2;  // left bound in use (every wl_ test is guarded by it)
    constexpr bool SPARSE = MASK == 3;
    // STREAM: the workgroup takes several items in a row (persistent
    // launch), its key tiles one stream through the stages.  Not with a
    // block map (its tile list is built once) and not at d = 256 (no
    // registers left for the next item's Q).
    constexpr bool MULTI = STREAM;
    static_assert(!STREAM || (!SPARSE && D <= 128), "streamed launches: no block map, d <= 128");
    const int wl_ = MASK >= 2 ? p.wl : kUnbounded;
    const int wr_ = MASK >= 2 ? p.wr : 0;
    constexpr int BN = pp_bn<D>();
    constexpr int NST = kPPStages;
    constexpr int BM = kPPBM;
    constexpr int TILE = BN * D;
    constexpr int KB = BN / 32;
    constexpr int QL = D / 16;  // Q loads of one item per lane
    using Copy = TileCopy<D, BN, kPPWaves>;
    constexpr int CPW = 2 * Copy::PER_WAVE;  // copy instructions per wave per tile
    static_assert((NST - 1) * CPW + QL <= 30, "vmcnt counts fit the wait helper");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int grp = w >> 2;                                  // 0: group A, 1: group B
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;  // > 0

    // ---- Items of this workgroup.  Ids follow fwd_decompose (heaviest
    // causal query blocks first, units ordered over the XCDs).  A launch with
    // fewer workgroups (G) than items (U) gives workgroup x the id x, then
    // one id of each further G-wide round; odd rounds run backwards over the
    // groups of 8 ids, so heavy and light causal blocks pair up while every
    // id keeps its residue mod 8 (G is a multiple of 8 then).  Every item of
    // such a launch has at least one tile (fixed lengths, no block map).
    // Wave 0 decodes the items into a table in LDS; the stream then reads
    // item k with two LDS loads.
    const int units = p.B * p.Hq;
    const int U = p.nqb * units;
    const int G = gridDim.x;
    const int wg = blockIdx.x;
    const bool multi = MULTI && G < U && p.cu == nullptr;
    auto item_id = [&](int k) -> int {
        if (k == 0) return wg;
        if (!multi) return U;
        if (!(k & 1)) return k * G + wg;
        return (k + 1) * G - 8 * (1 + (wg >> 3)) + (wg & 7);
    };
    auto decode = [&](int id, PPItem& it, int& bh) {
        int qb, b, h;
        fwd_decompose(id, units, p.nqb, p.Hq, CAUSAL, p.cu != nullptr, qb, b, h);
        const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
        it.qrow0 = sq.qrow(h);
        it.kvrow0 = sq.kvrow(h / (p.Hq / p.Hkv));
        it.qb = qb;
        it.n = sq.n;
        bh = b * p.Hq + h;
        const int q0 = qb * BM;
        // Masked kernels see keys q - wl .. q + wr of each query q (causal:
        // wl unbounded, wr = 0).
        const int kend = CAUSAL ? min(sq.n, q0 + BM + wr_) : sq.n;
        it.kt0 = WIN ? max(0, q0 - wl_) / BN : 0;
        it.T = q0 < sq.n ? (kend + BN - 1) / BN - it.kt0 : 0;
    };
    int* const tlist = reinterpret_cast<int*>(smem_raw + pp_lds_bytes<D>());
    PPItem* const table = reinterpret_cast<PPItem*>(smem_raw + pp_table_off<D, MASK>());
    int* const table_bh = reinterpret_cast<int*>(table + kPPItemCap);
    int* const table_tiles = table_bh + kPPItemCap;
    int nitems = 1;
    if constexpr (STREAM) {
        const int rounds = U / G;
        nitems = !multi ? 1 : min(kPPItemCap, rounds + (item_id(rounds) < U ? 1 : 0));
        if (w == 0) {
            int tiles = 0;
            for (int k = lane; k < nitems; k += 64) {
                PPItem it;
                decode(item_id(k), it, table_bh[k]);
                table[k] = it;
                tiles += it.T;
            }
            // total tiles of the stream
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) tiles += __shfl_xor(tiles, off);
            if (lane == 0) *table_tiles = tiles;
        }
        __syncthreads();
    }
    auto get_item = [&](int k, PPItem& it) {
        const u32x4 a = lds16(table + k);
        const u32x4 b2 = lds16(reinterpret_cast<const unsigned char*>(table + k) + 16);
        it.qrow0 = size_t(__builtin_amdgcn_readfirstlane(a[0])) | (size_t(__builtin_amdgcn_readfirstlane(a[1])) << 32);
        it.kvrow0 = size_t(__builtin_amdgcn_readfirstlane(a[2])) | (size_t(__builtin_amdgcn_readfirstlane(a[3])) << 32);
        it.qb = __builtin_amdgcn_readfirstlane(b2[0]);
        it.n = __builtin_amdgcn_readfirstlane(b2[1]);
        it.kt0 = __builtin_amdgcn_readfirstlane(b2[2]);
        it.T = __builtin_amdgcn_readfirstlane(b2[3]);
    };

    PPItem cur;  // the item this wave's compute is on
    int cur_bh;  // its batch * H_q + head
    int TT;      // key tiles of the whole stream
    if constexpr (STREAM) {
        get_item(0, cur);
        cur_bh = __builtin_amdgcn_readfirstlane(lds_i32(table_bh));
        TT = __builtin_amdgcn_readfirstlane(lds_i32(table_tiles));
    } else {
        decode(wg, cur, cur_bh);
        TT = cur.T;
    }
    if (cur.T == 0) return;  // past the end of a shorter packed sequence (whole workgroup)

    // Block-sparse (one item): the tiles of that range whose map block is
    // visible to group A (map row q0 / 128, tag bit 0) or group B (the next
    // row, bit 1), listed in LDS after the stages; a tile's local index then
    // indexes the list.
    if constexpr (SPARSE) {
        const int r0 = cur.qb * BM / kSparseBlock;
        const int kt0 = cur.kt0;
        if (w == 0) {
            const int cnt = compact_tiles(tlist, cur.T, lane, [&](int t) {
                const int col = (kt0 + t) * BN / kSparseBlock;
                return int(p.bmask[size_t(r0) * p.nb + col] != 0) |
                       (r0 + 1 < p.nb && p.bmask[size_t(r0 + 1) * p.nb + col] != 0 ? 2 : 0);
            });
            if (lane == 0) tlist[kSparseListCap] = cnt;
        }
        __syncthreads();
        cur.T = TT = __builtin_amdgcn_readfirstlane(lds_i32(tlist + kSparseListCap));
    }
    // First key of local tile j of item `it`, and (block-sparse) which
    // groups see it.
    auto tile_key0 = [&](const PPItem& it, int j) -> int {
        if constexpr (SPARSE) return (it.kt0 + (__builtin_amdgcn_readfirstlane(lds_i32(tlist + j)) & 0xFFFFFF)) * BN;
        else return (it.kt0 + j) * BN;
    };
    auto group_sees = [&](int j) -> bool {
        if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(lds_i32(tlist + j)) >> (24 + grp)) & 1;
        else return true;
    };

    // Q rows of an item as MFMA B operands (Q[row][16cc + 8hi .. +7]).  The
    // loads come first and alone (every lane loads: rows past the end read
    // the last row), so each call is exactly QL vector loads per wave and
    // nothing waits for them; fix_q then zeroes rows past the end and
    // applies qmode (1 negates: negative scale; 2 zeroes: zero scale)
    // without branches, once the data is needed.
    auto load_q = [&](bf16x8(&dst)[QL], const PPItem& it) {
        const int row = it.qb * BM + 32 * w + l32;
        const bf16* Qh = static_cast<const bf16*>(p.Q) + it.qrow0 * D + size_t(min(row, it.n - 1)) * D;
#pragma unroll
        for (int cc = 0; cc < QL; ++cc) dst[cc] = as_bf16x8(ld16(Qh + 16 * cc + 8 * hi));
    };
    auto fix_q = [&](bf16x8(&dst)[QL], const bf16x8(&src)[QL], int row, int n) {
        const uint32_t keep = (row < n && p.qmode != 2) ? 0xFFFFFFFFu : 0u;
        const uint32_t neg = p.qmode == 1 ? 0x80008000u : 0u;
#pragma unroll
        for (int cc = 0; cc < QL; ++cc) {
            const u32x4 v = as_u32x4(src[cc]);
            dst[cc] = as_bf16x8(u32x4{(v[0] & keep) ^ neg, (v[1] & keep) ^ neg, (v[2] & keep) ^ neg,
                                      (v[3] & keep) ^ neg});
        }
    };

    // ---- Copies: one cursor walks the stream's tiles in order (global tile
    // t goes to stage t % NST).
    Copy cp;
    cp.init(w, lane);
    PPItem iss = cur;  // item of the next tile to copy
    int iss_k = 0, iss_j = 0;
    auto issue_next = [&](int t) {
        if constexpr (!STREAM) {
            // one item: global tile t is its local tile t
            bf16* st = smem + (t % NST) * 2 * TILE;
            cp.issue(static_cast<const bf16*>(p.K) + cur.kvrow0 * D, static_cast<const bf16*>(p.V) + cur.kvrow0 * D,
                     st, st + TILE, tile_key0(cur, t), cur.n);
            return;
        }
        if (iss_j == iss.T) {
            ++iss_k;
            get_item(iss_k, iss);
            iss_j = 0;
        }
        const bf16* Kh = static_cast<const bf16*>(p.K) + iss.kvrow0 * D;
        const bf16* Vh = static_cast<const bf16*>(p.V) + iss.kvrow0 * D;
        bf16* st = smem + (t % NST) * 2 * TILE;
        cp.issue(Kh, Vh, st, st + TILE, tile_key0(iss, iss_j), iss.n);
        ++iss_j;
    };

    // Q of the first item (the oldest loads of the wave), then the prologue
    // tiles 0 .. min(TT, NST) - 1 into the empty stages.
    bf16x8 qreg[QL];
    bf16x8 qnext[MULTI ? QL : 1];  // the next item's Q, loaded ahead
    if constexpr (STREAM) {
        load_q(qreg, cur);
    } else {
        const int row = cur.qb * BM + 32 * w + l32;
        const bf16* Qh = static_cast<const bf16*>(p.Q) + cur.qrow0 * D;
#pragma unroll
        for (int cc = 0; cc < QL; ++cc) {
            u32x4 v = u32x4{0, 0, 0, 0};
            if (row < cur.n && p.qmode != 2) v = ld16(Qh + size_t(row) * D + 16 * cc + 8 * hi);
            if (p.qmode == 1) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            qreg[cc] = as_bf16x8(v);
        }
    }
#pragma unroll
    for (int t = 0; t < NST; ++t)
        if (t < TT) issue_next(t);

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

    // Compute view: rows of this wave in the current item.
    int cur_k = 0, cur_start = 0;  // item counter, global index of its first tile
    int wq0, wq_last, qrow, key_lim, key_lo;
    auto set_view = [&]() {
        wq0 = cur.qb * BM + 32 * w;  // first query row of this wave (uniform)
        wq_last = wq0 + 31;
        qrow = wq0 + l32;
        key_lim = CAUSAL ? min(qrow + wr_, cur.n - 1) : cur.n - 1;  // last visible key of this row
        key_lo = WIN ? qrow - wl_ : 0;                              // first visible key
    };
    set_view();

    // Number of 32-key blocks of global tile g (of the current item) this
    // wave must process (uniform).
    auto active_kb = [&](int g) -> int {
        if (!CAUSAL) return KB;
        const int j = g - cur_start;
        if (!group_sees(j)) return 0;
        const int kstart = tile_key0(cur, j);
        if (kstart > wq_last + wr_ || (WIN && kstart + BN - 1 < wq0 - wl_)) return 0;
        return min(KB, (wq_last + wr_ - kstart) / 32 + 1);
    };

    // Tile 0 must be in LDS before step 0: wait for it (the newer prologue
    // tiles may stay in flight), then publish.
    wait_vmem_at_most<CPW>(min(TT, NST) - 1);
    __syncthreads();
    if constexpr (STREAM) fix_q(qreg, qreg, qrow, cur.n);

    // Steps 0 .. 2TT+1, one workgroup barrier after each.  Group A: step 2j
    // is its M phase j, step 2j+1 its V phase j.  Group B runs one step
    // later.  Refill: at even step 2u (u >= 2) tile u + 2 goes into the
    // stage of tile u - 2, whose last reader (group B, M phase u - 1: the V
    // operand of tile u - 2) finished at the previous barrier.
    auto copies_at = [&](int step) -> int {
        return (!(step & 1) && step >= 4 && step / 2 + 2 < TT) ? CPW : 0;
    };
    auto refill = [&](int step) {
        if (copies_at(step)) issue_next(step / 2 + 2);
    };
    bool qpend = false;  // the next item's Q loads are in flight
    // End of a step: before step 2t (group A reads K_t) every wave has
    // waited for its own copies of tile t.  At the end of step 2t - 1 the
    // tiles issued so far are 0 .. max(NST - 1, t + 1) (bounded by TT - 1);
    // Q loads issued after tile t's copies and not yet used are newer too.
    auto finish = [&](int step) {
        if (step & 1) {
            const int t = (step + 1) / 2;
            if (t < TT) {
                const int n = min(TT - 1, max(NST - 1, t + 1)) - t;  // tiles issued after t
                if constexpr (STREAM) wait_vmcnt(CPW * n + (qpend ? QL : 0));
                else wait_vmem_at_most<CPW>(n);
            }
        }
        wait_lds();  // this wave's LDS reads are done before the stage can be refilled
        __builtin_amdgcn_s_barrier();
    };

    // Output of the finished item: O = o / l (bf16), LSE = m + log2 l
    // (natural log); then the accumulators start over.
    // O rows leave the wave in one of two ways.  At the end of a launch of
    // one item per workgroup the stages are free: every wave stages its 32
    // rows in LDS and stores whole rows, 16 bytes per lane.  Between items of
    // a persistent launch (the stages busy), the two halves of the wave trade
    // 8-byte chunks so that each lane stores 16 contiguous bytes of its row.
    auto epilogue = [&](auto staged) {
        const float lt = half_swap_sum(l);
        // A row that sees no key at all (block-sparse only) has l = 0: O = 0,
        // LSE = -inf.  Dropout scales the kept terms by 256 / (256 - t8).
        float inv = (!SPARSE || lt > 0.f) ? 1.f / lt : 0.f;
        if constexpr (DROP) inv *= 256.f / float(256 - p.drop_t8);
        if constexpr (decltype(staged)::value) {
            static_assert(kPPWaves * staged_rows_bytes<D, bf16>() <= int(pp_lds_bytes<D>()), "staging must fit");
            store_rows_staged<D>(smem_raw + w * staged_rows_bytes<D, bf16>(), o, inv,
                                 static_cast<bf16*>(p.O) + (cur.qrow0 + size_t(wq0)) * D, cur.n - wq0, lane);
        } else if (qrow < cur.n) {
            bf16* orow = static_cast<bf16*>(p.O) + (cur.qrow0 + size_t(qrow)) * D;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
#pragma unroll
                for (int jj = 0; jj < 4; jj += 2) {
                    if constexpr (D == 64) {  // measured: the trade does not pay for 128-byte rows
                        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * jj + 4 * hi) =
                            bf16x4{(bf16)(o[db][4 * jj + 0] * inv), (bf16)(o[db][4 * jj + 1] * inv),
                                   (bf16)(o[db][4 * jj + 2] * inv), (bf16)(o[db][4 * jj + 3] * inv)};
                        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * jj + 8 + 4 * hi) =
                            bf16x4{(bf16)(o[db][4 * jj + 4] * inv), (bf16)(o[db][4 * jj + 5] * inv),
                                   (bf16)(o[db][4 * jj + 6] * inv), (bf16)(o[db][4 * jj + 7] * inv)};
                        continue;
                    }
                    // half 0 ends with dims 8jj .. 8jj+7 of its row, half 1 with 8jj+8 .. 8jj+15
                    const bf16x4 a = bf16x4{(bf16)(o[db][4 * jj + 0] * inv), (bf16)(o[db][4 * jj + 1] * inv),
                                            (bf16)(o[db][4 * jj + 2] * inv), (bf16)(o[db][4 * jj + 3] * inv)};
                    const bf16x4 b = bf16x4{(bf16)(o[db][4 * jj + 4] * inv), (bf16)(o[db][4 * jj + 5] * inv),
                                            (bf16)(o[db][4 * jj + 6] * inv), (bf16)(o[db][4 * jj + 7] * inv)};
                    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
                    u32x2 y;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int x = int(hi ? ua[e] : ub[e]);
                        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
                        y[e] = uint32_t(hi ? r[0] : r[1]);
                    }
                    const u32x4 v = hi ? u32x4{y[0], y[1], ub[0], ub[1]} : u32x4{ua[0], ua[1], y[0], y[1]};
                    *reinterpret_cast<u32x4*>(orow + db * 32 + 8 * (jj + hi)) = v;
                }
            }
        }
        if (qrow < cur.n && hi == 0 && p.LSE != nullptr)
            p.LSE[cur.qrow0 + qrow] = (!SPARSE || lt > 0.f) ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
        m = -3.0e38f;
        l = 0.f;
    };
    // ---- Item switches, in the M phase of the first tile g of the next item
    // (group A at step 2g, group B at 2g + 1), after the PV of tile g - 1
    // and the epilogue: the next item's Q, loaded into qnext two steps
    // earlier, becomes qreg and the view moves on.
    auto switch_item = [&](int g, int step) {
        if constexpr (MULTI) {
            // loads issued after the Q loads: this group's copies at the step after them
            wait_vmcnt(copies_at(grp == 0 ? step - 2 : step - 1));
            qpend = false;
            ++cur_k;
            get_item(cur_k, cur);
            cur_bh = __builtin_amdgcn_readfirstlane(lds_i32(table_bh + cur_k));
            cur_start = g;
            set_view();
            fix_q(qreg, qnext, qrow, cur.n);
        }
    };
    // If g is the last tile of its item, the Q of the item after it goes to
    // qnext: before this step's copies (group A) or in a step without copies
    // (group B), so the wave's queue holds them in that order.  Every M
    // phase runs PV, [epilogue, switch], this, the step's copies, QK: the
    // compiler's own wait before the first read of qnext (it does not count
    // the direct-to-LDS copies) then only covers copies a step old.
    auto prefetch_q = [&](int g) {
        if constexpr (MULTI) {
            if (g < TT && g == cur_start + cur.T - 1 && cur_k + 1 < nitems) {
                PPItem nx;
                get_item(cur_k + 1, nx);
                load_q(qnext, nx);
                qpend = true;
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    int akb_pv = 0;  // 32-key blocks of the tile whose PV comes next (computed with its item's view)
    // ---- M phase g: PV of tile g-1, then QK of tile g.  LDS fragments are
    // loaded one block ahead of the MFMAs that use them; scheduling barriers
    // keep at most two blocks live.
    auto pv = [&](int g) {
        if (g >= 1 && akb_pv > 0) {
            // V^T A operand of contraction block (kb, cc): keys
            // 32kb + 16cc + 8(sl/4) + 4hi + sl%4 of dims db*32 + l32, read
            // transposed from the V slabs of tile g-1.
            const bf16* Vs = smem + ((g - 1) % NST) * 2 * TILE + TILE;
            // Chunks of VC output dim blocks, in the order (kb, cc, chunk);
            // chunk x + 1 is loaded while the MFMAs of chunk x run.
            constexpr int VC = D / 32 > 4 ? 1 : (STREAM && D / 32 > 2) ? 2 : D / 32;
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
    };
    auto qk = [&](int g) {
        akb_pv = g < TT ? active_kb(g) : 0;
        if (akb_pv > 0) {
            const bf16* Ks = smem + (g % NST) * 2 * TILE;
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
    // The M phase of tile g at `step`, with the step's copies.  An item
    // ends after the PV of its last tile (g - 1): epilogue, then the switch
    // to the next item before its first QK.
    // The group in its M phase issues at raised wave priority, so that the
    // other group's softmax instructions fill the gaps between its matrix
    // products rather than delay them (d >= 128: 0.5-3 % faster; d = 64, where
    // a phase has half the products, 2 % slower).
    auto phase_m = [&](int g, int step) {
        if constexpr (D >= 128) __builtin_amdgcn_s_setprio(1);
        if constexpr (STREAM) {
            pv(g);
            if (g == cur_start + cur.T) {
                epilogue(std::false_type{});
                if (g < TT) switch_item(g, step);
            }
            prefetch_q(g);
            refill(step);
        } else {
            // one item: the copies first in the step, the epilogue after the loop
            refill(step);
            pv(g);
        }
        qk(g);
        if constexpr (D >= 128) __builtin_amdgcn_s_setprio(0);
    };
    // ---- V phase g: online softmax of S_g -> P_g (bf16), O rescaled if needed.
    auto phase_v = [&](int g) {
        if (g >= TT || akb_pv == 0) return;
        const int kstart = tile_key0(cur, g - cur_start);
        const bool mask_hi = (CAUSAL && kstart + BN - 1 > wq0 + wr_) || (kstart + BN > cur.n);
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
                drop_bytes_qmajor(y, qrow, kstart + 32 * kb, hi, lane, uint32_t(cur_bh), p.drop_off,
                                  p.drop_k0, p.drop_k1);
#pragma unroll
                for (int r = 0; r < 16; ++r) e[r] = drop_keep(y, r, p.drop_t8) ? e[r] : 0.f;
            }
            pb[kb][0] = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
            pb[kb][1] = to_bf16x8(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
        }
        l += rs;
    };

    if (grp == 0) {
        for (int g = 0; g <= TT; ++g) {
            phase_m(g, 2 * g);
            finish(2 * g);
            refill(2 * g + 1);
            phase_v(g);
            finish(2 * g + 1);
        }
    } else {
        finish(0);
        for (int g = 0; g <= TT; ++g) {
            phase_m(g, 2 * g + 1);
            finish(2 * g + 1);
            if (g < TT) {
                refill(2 * g + 2);
                phase_v(g);
                finish(2 * g + 2);
            }
        }
    }
    if constexpr (!STREAM) {
        // Both groups end on the same barrier, each wave having drained its
        // LDS reads before it and every copy having landed before the last
        // tile was published: the stages are free for staging rows.  (At
        // d = 256 staging through LDS costs registers the kernel has not got.)
        if constexpr (D <= 128) epilogue(std::true_type{});
        else epilogue(std::false_type{});
    }
}

// Persistent launch (fixed lengths, no block map, d <= 128) when a query
// block's key tiles are few (causal N up to 4096 - 256, non-causal up to
// 2048, windows): one workgroup per compute unit (the LDS holds one) walks
// several items, so the per-workgroup start (Q and the first tiles) and the
// pipeline fill and drain are paid once per compute unit.  Longer blocks
// keep one workgroup per item (their start is a small share, and
// workgroups that start together share key/value tiles in the L2).
template <int D, int MASK>
bool use_stream(const FwdParams& p, long long items, int cus) {
    if (MASK == 3 || D > 128 || p.cu != nullptr || cus % 8 != 0 || items <= cus) return false;
    const int nkt = (p.N + 63) / 64;  // 64-key tiles of the whole sequence
    double avg;                        // average 64-key tiles per query block
    if (MASK == 0) avg = nkt;
    else if (MASK == 1) avg = 0.5 * (nkt + 4.0);
    else avg = double(min(p.N, (p.wl >= kUnbounded ? p.N : p.wl) + (p.wr >= kUnbounded ? p.N : p.wr) + kPPBM)) / 64.0;
    return avg <= 32.0;
}

template <int D, int MASK, bool DROP = false>
hipError_t launch_fwd_pp_t(FwdParams p, hipStream_t stream) {
    p.nqb = (p.N + kPPBM - 1) / kPPBM;
    long long blocks = (long long)p.nqb * p.B * p.Hq;
    const int cus = device_cu_count();
    if constexpr (MASK != 3 && D <= 128) {
        if (use_stream<D, MASK>(p, blocks, cus)) {
            auto kern = fwd_pp_kernel<D, MASK, DROP, true>;
            constexpr size_t lds = pp_lds_total<D, MASK, true>();
            static DeviceOnce attr;
            const hipError_t e = set_max_dynamic_lds(kern, lds, attr);
            if (e != hipSuccess) return e;
            // at most kPPItemCap items per workgroup: more workgroups (a multiple of 8) when needed
            long long g = (blocks + kPPItemCap - 1) / kPPItemCap;
            g = (g + 7) / 8 * 8;
            g = g > cus ? g : cus;
            hipLaunchKernelGGL(kern, dim3(unsigned(g)), dim3(kPPWaves * 64), lds, stream, p);
            return hipGetLastError();
        }
    }
    auto kern = fwd_pp_kernel<D, MASK, DROP, false>;
    constexpr size_t lds = pp_lds_total<D, MASK, false>();
    static DeviceOnce attr;
    const hipError_t e = set_max_dynamic_lds(kern, lds, attr);
    if (e != hipSuccess) return e;
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
