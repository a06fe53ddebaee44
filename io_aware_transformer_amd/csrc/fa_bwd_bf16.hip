// Backward pass, bf16 inputs, fp32 accumulation, gfx950 matrix cores.
//
// The scores are recomputed on chip from Q, K and the saved per-row LSE
// instead of being stored ("The Future of AI: How FlashAttention
// Revolutionizes Deep Learning", "Understanding FlashAttention",
// recomputation bullet).  The pages print no backward formulas; the kernels
// evaluate the analytic derivative of O = softmax(scale Q K^T) V:
//   P = exp(scale S - LSE), dV = P^T dO, dP = dO V^T,
//   D_i = sum_j P_ij dP_ij = dO_i . O_i, dS = P o (dP - D),
//   dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels on the caller's stream:
//   1. bwd_pre:  D_i = dO_i . O_i (fp32, into the workspace).
//   2. bwd_dkdv: one workgroup per (batch, kv head, block of keys); each
//      wave keeps its keys' K and V rows in registers and its dK, dV
//      accumulators in registers, and walks every query tile (of every
//      query head of the group) that can see its keys.  S = Q K^T and
//      dP = dO V^T come out with one key per lane, which is exactly the MFMA
//      A layout of P^T and dS^T, so dV += P^T dO and dK += dS^T Q take the
//      score registers directly; dO and Q enter as B operands through
//      transposing LDS reads.  dK, dV are written once: no atomics.
//      v2 keeps two 32-key blocks per wave (d = 64); v3 is software-
//      pipelined with one block per wave (d = 128).
//   3. bwd_dq:   one workgroup per (batch, query head, 256 queries), 64 rows
//      per wave: S^T = K Q^T, dP^T = V dO^T with one query per lane,
//      dQ^T += K^T dS^T with K^T through transposing LDS reads.
// Splitting dQ from dK/dV recomputes S and dP once more (7 matrix products
// instead of 5) but needs no fp32 dQ accumulator and no atomic traffic.
// The masked kernels (MASK 1: causal, 2: a window (wl, wr)) visit only the
// tiles a window can see and mask the scores of the edge tiles.
#include "fa_device.hpp"
#include "fa_internal.h"

#include <math.h>

#include <type_traits>

namespace fa {

// Fixed device buffer of the allocation-free backward (fa_bwd_noalloc): it
// holds the D_i term in place of a caller workspace.  Every device the
// library runs on keeps one copy for the life of the process; calls on one
// device share it (and race when they overlap).
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void* noalloc_scratch(hipError_t& err) {
    // The host-side name `scratch` is only a handle: its device address,
    // different on every device, comes from hipGetSymbolAddress, taken once
    // per device with that device current.
    static std::atomic<void*> addr[64];
    int dev = 0;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= 64) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    void* ptr = addr[dev].load(std::memory_order_acquire);
    if (ptr != nullptr) return ptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return nullptr;
    addr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

namespace {

__device__ __forceinline__ f32x4 lds_free_ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// ---------------------------------------------------------------- bwd_pre
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                      float* __restrict__ Drow, long long rows) {
    constexpr int LPR = D / 8;      // lanes per row, 8 elements each
    constexpr int RPB = 256 / LPR;  // rows per workgroup
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int part = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 o = as_bf16x8(ld16(O + row * D + 8 * part));
        const bf16x8 g = as_bf16x8(ld16(dO + row * D + 8 * part));
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf(float(o[i]), float(g[i]), acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && part == 0) Drow[row] = acc;
}


// ---------------------------------------------------------------- dK/dV slice sum
// dK = sum over the query-head slices of their float partials, in slice
// order (deterministic), rounded once to bf16; 4 elements per thread.
__global__ __launch_bounds__(256) void dkdv_reduce_kernel(const float* __restrict__ dkp, const float* __restrict__ dvp,
                                                          bf16* __restrict__ dK, bf16* __restrict__ dV, long long n4,
                                                          int S, size_t stride) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 k = lds_free_ld4(dkp + 4 * i), v = lds_free_ld4(dvp + 4 * i);
    for (int s = 1; s < S; ++s) {
        k += lds_free_ld4(dkp + s * stride + 4 * i);
        v += lds_free_ld4(dvp + s * stride + 4 * i);
    }
    *reinterpret_cast<bf16x4*>(dK + 4 * i) = bf16x4{(bf16)k[0], (bf16)k[1], (bf16)k[2], (bf16)k[3]};
    *reinterpret_cast<bf16x4*>(dV + 4 * i) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// ---------------------------------------------------------------- bwd_dkdv v2
// One workgroup of NW waves per (batch, kv head, block of 32*KPW*NW keys);
// each wave keeps KPW blocks of 32 keys (K and V rows as MFMA B operands)
// and their dK, dV accumulators.  Query tiles of 64 rows (Q, dO in padded K
// slabs, LSE and D) are copied global -> LDS by buffer loads, four stages,
// three tiles ahead (2-3 % faster than three stages at d = 64).  KPW = 2
// would let every Q / dO fragment read from LDS feed
// two products; at d = 64, 8 waves of one block each (two per SIMD, one
// wave's exponentials and dS under the other's matrix products) measured
// 7-10 % faster.  The accumulators are touched by the matrix cores only
// until the epilogue.
template <int D>
struct DkCfg;
template <>
struct DkCfg<64> {
    static constexpr int KPW = 1, NW = 8;
};
template <>
struct DkCfg<128> {
    static constexpr int KPW = 1, NW = 4;
};
constexpr int kDkWaves = 4;
constexpr int kDkBQ = 64;
constexpr int kDkStages = 4;

template <int D>
struct DkLds {
    using QL = PadSlab<kDkBQ, D>;
    static constexpr int TILE_BYTES = QL::ELEMS * 2;
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * kDkBQ * 4;
    static constexpr size_t BYTES = size_t(kDkStages) * STAGE_BYTES;
    static_assert(STAGE_BYTES % 16 == 0, "stage must keep 16-byte alignment");
};

template <int D>
constexpr int dk_keys_per_wg() {
    return 32 * DkCfg<D>::KPW * DkCfg<D>::NW;
}

template <int D, int MASK, bool DROP>
__global__ __launch_bounds__(DkCfg<D>::NW * 64) __attribute__((amdgpu_waves_per_eu(DkCfg<D>::NW / 4, DkCfg<D>::NW / 4)))
void bwd_dkdv2_kernel(BwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK == 2;  // left bound in use (every wl_ test is guarded by it)
    const int wl_ = MASK == 2 ? p.wl : kUnbounded;
    const int wr_ = MASK == 2 ? p.wr : 0;
    constexpr int KPW = DkCfg<D>::KPW;
    using QL = typename DkLds<D>::QL;
    constexpr int TB = DkLds<D>::TILE_BYTES;
    constexpr int SB = DkLds<D>::STAGE_BYTES;
    constexpr int NST = kDkStages;
    constexpr int BQ = kDkBQ;
    constexpr int NW = DkCfg<D>::NW;
    constexpr int PPW = QL::PIECES / NW;  // copy pieces per wave per matrix
    static_assert(QL::PIECES % NW == 0, "pieces must split over the waves");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;
    // unit = (batch, kv head, slice of its group's query heads)
    const int S = p.hsplit, Hs = p.Hkv * S;
    const int units = p.B * Hs;
    const int slot = blockIdx.x / units;
    const int unit = order_unit(blockIdx.x - slot * units, units, Hs, p.cu != nullptr);
    const int b = unit / Hs, gs = unit - (unit / Hs) * Hs;
    const int g = gs / S, sl = gs - (gs / S) * S;
    const int G = p.Hq / p.Hkv;
    const int GS = G / S;            // query heads of this workgroup
    const int h0 = g * G + sl * GS;  // the first of them
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    const int kstart = slot * dk_keys_per_wg<D>();
    if (kstart >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const int kw0 = kstart + 32 * KPW * w;  // first key of this wave (uniform)

    const size_t kvoff = sq.kvrow(g) * D;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;

    bf16x8 kreg[KPW][D / 16], vreg[KPW][D / 16];
    f32x16 dk[KPW][D / 32], dv[KPW][D / 32];
#pragma unroll
    for (int kb = 0; kb < KPW; ++kb) {
        const int key = kw0 + 32 * kb + l32;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            if (key < N) {
                kreg[kb][cc] = as_bf16x8(ld16(Kh + size_t(key) * D + 16 * cc + 8 * hi));
                vreg[kb][cc] = as_bf16x8(ld16(Vh + size_t(key) * D + 16 * cc + 8 * hi));
            } else {
                kreg[kb][cc] = bf16x8{};
                vreg[kb][cc] = bf16x8{};
            }
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
            dk[kb][db] = f32x16{};
            dv[kb][db] = f32x16{};
        }
    }

    // Query tiles that can see a key of this workgroup: queries k - wr .. k + wl
    // of each key k (masked kernels; causal: wr = 0, wl unbounded).
    const int nqt = (N + BQ - 1) / BQ;
    const int qt_first = CAUSAL ? max(0, kstart - wr_) / BQ : 0;
    const int qt_last = WIN ? min(nqt - 1, (kstart + dk_keys_per_wg<D>() - 1 + wl_) / BQ) : nqt - 1;
    const int per_head = qt_last - qt_first + 1;
    const int iters = GS * per_head;

    // Per-lane copy sources: piece pi = w + 4 i of the Q (and dO) tile.
    int src_off[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        int r, e0;
        QL::piece_src(w + NW * i, lane, r, e0);
        src_off[i] = r * D + e0;
    }
    auto issue = [&](int t) {
        const int hq = h0 + t / per_head;
        const int q0 = (qt_first + t % per_head) * BQ;
        const size_t row0 = sq.qrow(hq) + q0;
        unsigned char* st = smem_raw + (t % NST) * SB;
        const uint32_t bytes = uint32_t(N - q0) * uint32_t(D * 2);
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(static_cast<const bf16*>(p.Q) + row0 * D, bytes);
        const __amdgpu_buffer_rsrc_t orr = make_rsrc(static_cast<const bf16*>(p.dO) + row0 * D, bytes);
        const bool tail = q0 + BQ > N;
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int pi = w + NW * i;
            uint32_t off = uint32_t(src_off[i]);
            if (tail) off = uint32_t(min(src_off[i] / D, N - 1 - q0) * D + src_off[i] % D);
            buf16_to_lds(qr, 2 * off, st + 2 * QL::piece_dst(pi));
            buf16_to_lds(orr, 2 * off, st + TB + 2 * QL::piece_dst(pi));
        }
        // LSE and D of the 64 rows: 256 bytes each, lanes 0..15 of waves 0 / 1.
        if (w < 2 && lane < 16) {
            const float* src = (w == 0 ? p.LSE : p.Drow) + row0;
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(src, uint32_t(N - q0) * 4u);
            buf16_to_lds(rr, uint32_t(16 * lane), st + 2 * TB + w * BQ * 4);
        }
    };
    // s_waitcnt vmcnt: the `ahead` tiles issued after the next one stay in flight
    // (this wave's copies per tile: 2 PPW, plus the statistics in waves 0 and 1).
    auto wait_older = [&](int ahead) {
        if (ahead >= 2) {
            if (w < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * PPW + 2) & 15) | (((4 * PPW + 2) >> 4) << 14));
            else __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * PPW) & 15) | (((4 * PPW) >> 4) << 14));
        } else if (ahead == 1) {
            if (w < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PPW + 1) & 15) | (((2 * PPW + 1) >> 4) << 14));
            else __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PPW) & 15) | (((2 * PPW) >> 4) << 14));
        } else {
            wait_vmem();
        }
    };

    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (iters > 0) issue(0);
    if (iters > 1) issue(1);
    if (iters > 2) issue(2);
    wait_vmem();
    __syncthreads();

    for (int t = 0; t < iters; ++t) {
        if (t + 3 < iters) issue(t + 3);
        const unsigned char* st = smem_raw + (t % NST) * SB;
        const bf16* Qs = reinterpret_cast<const bf16*>(st);
        const bf16* dOs = reinterpret_cast<const bf16*>(st + TB);
        const float* ls = reinterpret_cast<const float*>(st + 2 * TB);
        const float* dsr = ls + BQ;
        const int q0 = (qt_first + t % per_head) * BQ;

#pragma unroll
        for (int qs = 0; qs < BQ / 32; ++qs) {
            const int qb0 = q0 + 32 * qs;
            // Skip the subtile when no key block of this wave sees any of its
            // rows; otherwise compute every block (a block that sees none is
            // wholly hidden by the mask below and adds zeros), which keeps the
            // matrix-core code free of branches.
            bool any = false;
#pragma unroll
            for (int kb = 0; kb < KPW; ++kb) {
                const int key0 = kw0 + 32 * kb;
                any = any || ((!CAUSAL || (qb0 + 31 >= key0 - wr_ && (!WIN || qb0 <= key0 + 31 + wl_))) && qb0 < N);
            }
            if (!any) continue;
            // S = Q K^T, dP = dO V^T: lane = key, register r = query qb0 + 8(r/4) + 4hi + r%4
            f32x16 sacc[KPW], dpacc[KPW];
#pragma unroll
            for (int kb = 0; kb < KPW; ++kb) sacc[kb] = dpacc[kb] = f32x16{};
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                const bf16x8 aq = as_bf16x8(lds16(Qs + QL::off(32 * qs + l32, 16 * cc + 8 * hi)));
                const bf16x8 ao = as_bf16x8(lds16(dOs + QL::off(32 * qs + l32, 16 * cc + 8 * hi)));
#pragma unroll
                for (int kb = 0; kb < KPW; ++kb) {
                    sacc[kb] = mfma_32x32x16(aq, kreg[kb][cc], sacc[kb]);
                    dpacc[kb] = mfma_32x32x16(ao, vreg[kb][cc], dpacc[kb]);
                }
            }
            float lq[16], dq[16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 lv = lds_f32x4(ls + 32 * qs + 8 * j + 4 * hi);
                const f32x4 dv4 = lds_f32x4(dsr + 32 * qs + 8 * j + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lq[4 * j + e] = lv[e] * kLog2e;
                    dq[4 * j + e] = dv4[e];
                }
            }
            bf16x8 pb[KPW][2], sb[KPW][2];
#pragma unroll
            for (int kb = 0; kb < KPW; ++kb) {
                float pr[16], ds[16];
                const int key0 = kw0 + 32 * kb;
                if constexpr (DROP) {
                    // Dropout: P enters dV dropped (its 256 / (256 - t8)
                    // factor is applied to dV at the end); dP = dO V^T is
                    // dropped and scaled before dS.
                    uint32_t dy[4];
                    drop_bytes_kmajor(dy, key0 + l32, qb0, hi, lane, uint32_t(b * p.Hq + h0 + t / per_head),
                                      p.drop_off, p.drop_k0, p.drop_k1);
                    const float dinv = 256.f / float(256 - p.drop_t8);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const bool kp = drop_keep(dy, r, p.drop_t8);
                        pr[r] = fast_exp2(fmaf(sacc[kb][r], c, -lq[r]));
                        ds[r] = pr[r] * ((kp ? dpacc[kb][r] * dinv : 0.f) - dq[r]);
                        pr[r] = kp ? pr[r] : 0.f;
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        pr[r] = fast_exp2(fmaf(sacc[kb][r], c, -lq[r]));
                        ds[r] = pr[r] * (dpacc[kb][r] - dq[r]);
                    }
                }
                if ((CAUSAL && (qb0 < key0 + 31 - wr_ || (WIN && qb0 + 31 > key0 + wl_))) || qb0 + 31 >= N) {
                    // hide queries outside key - wr .. key + wl and rows q >= N: P and dS become 0
                    const int thr = CAUSAL ? key0 + l32 - wr_ - qb0 - 4 * hi : -1;
                    const int thr_hi = WIN ? key0 + l32 + wl_ - qb0 - 4 * hi : kUnbounded;
                    const int nlim = N - qb0 - 4 * hi;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qo = 8 * (r >> 2) + (r & 3);
                        const bool hide = (qo < thr) || (qo > thr_hi) || (qo >= nlim);
                        pr[r] = hide ? 0.f : pr[r];
                        ds[r] = hide ? 0.f : ds[r];
                    }
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    pb[kb][cc] = to_bf16x8(pr[8 * cc + 0], pr[8 * cc + 1], pr[8 * cc + 2], pr[8 * cc + 3], pr[8 * cc + 4],
                                           pr[8 * cc + 5], pr[8 * cc + 6], pr[8 * cc + 7]);
                    sb[kb][cc] = to_bf16x8(ds[8 * cc + 0], ds[8 * cc + 1], ds[8 * cc + 2], ds[8 * cc + 3], ds[8 * cc + 4],
                                           ds[8 * cc + 5], ds[8 * cc + 6], ds[8 * cc + 7]);
                }
            }
            // dV^T += dO^T P, dK^T += Q^T dS: dO and Q enter as A operands
            // through transposing reads, each fragment feeding KPW products
            // (the transposed products leave one key per lane).
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int qr = 32 * qs + 16 * cc + trow;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 bo = cat(lds_read_tr(dOs + QL::off(qr, db * 32 + tcol)),
                                          lds_read_tr(dOs + QL::off(qr + 8, db * 32 + tcol)));
                    const bf16x8 bq = cat(lds_read_tr(Qs + QL::off(qr, db * 32 + tcol)),
                                          lds_read_tr(Qs + QL::off(qr + 8, db * 32 + tcol)));
#pragma unroll
                    for (int kb = 0; kb < KPW; ++kb) {
                        dv[kb][db] = mfma_32x32x16(bo, pb[kb][cc], dv[kb][db]);
                        dk[kb][db] = mfma_32x32x16(bq, sb[kb][cc], dk[kb][db]);
                    }
                }
            }
        }
        // This wave's copies of the next tile are done once only those of the
        // tiles issued after it remain; drain this wave's LDS reads (the stage
        // just read is refilled next) and meet at a plain barrier: a
        // __syncthreads() fence would also wait for the newer copies.
        wait_older(min(iters - 1, t + 3) - (t + 1));
        barrier_lds();
    }

    // Epilogue: lane holds key kw0 + 32kb + l32, dims db*32 + 8(r/4) + 4hi + r%4;
    // whole rows through this wave's LDS region.
    const float vscale = DROP ? 256.f / float(256 - p.drop_t8) : 1.f;
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < KPW; ++kb) {
        const int k0 = kw0 + 32 * kb;
        const size_t row0 = kvoff + size_t(k0) * D;
        if (S == 1) {
            static_assert(NW * staged_rows_bytes<D, bf16>() <= int(DkLds<D>::BYTES), "staging must fit");
            unsigned char* stg = smem_raw + w * staged_rows_bytes<D, bf16>();
            store_rows_staged<D>(stg, dk[kb], p.scale, static_cast<bf16*>(p.dK) + row0, N - k0, lane);
            store_rows_staged<D>(stg, dv[kb], vscale, static_cast<bf16*>(p.dV) + row0, N - k0, lane);
        } else {
            static_assert(NW * staged_rows_bytes<D, float>() <= int(DkLds<D>::BYTES), "staging must fit");
            unsigned char* stg = smem_raw + w * staged_rows_bytes<D, float>();
            store_rows_staged<D>(stg, dk[kb], p.scale, p.dk_part + sl * p.part_stride + row0, N - k0, lane);
            store_rows_staged<D>(stg, dv[kb], vscale, p.dv_part + sl * p.part_stride + row0, N - k0, lane);
        }
    }
}

// ---------------------------------------------------------------- bwd_dkdv v3
// Software-pipelined key-major dK / dV, one wave per SIMD, 32 keys per wave,
// query subtiles of 32 rows (two per staged 64-row tile).  Subtile i passes
// through three steps: A(i) S = Q K^T, dP = dO V^T (matrix cores, row reads
// of Q / dO issued one step ahead); B(i) P = exp2(c S - LSE log2 e),
// dS = P o (dP - D) (vector ALU); C(i) dV^T += dO^T P, dK^T += Q^T dS
// (matrix cores, transposing reads of dO / Q; the transposed products leave
// one key per lane, so the epilogue stores whole rows).  The loop body for subtile i runs
// A(i+1) together with B(i) and the transposing reads of C(i), then C(i)
// together with the row reads for A(i+2): every LDS read has a whole step
// of slack before its first use, and the LDS traffic is split evenly over
// the two steps.  (Vector ALU work of a wave overlaps that wave's own
// matrix-core work only partly on this chip; the gain is the hidden LDS
// latency.)  Four stages of 64-row tiles; tile t+3 is issued right after
// the barrier that publishes tile t+1.  Used for d = 128.
constexpr int kDk3Stages = 4;

template <int D>
struct Dk3Lds {
    using QL = PadSlab<kDkBQ, D>;
    static constexpr int TILE_BYTES = QL::ELEMS * 2;
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES + 2 * kDkBQ * 4;
    static constexpr size_t BYTES = size_t(kDk3Stages) * STAGE_BYTES;
    static_assert(STAGE_BYTES % 16 == 0, "stage must keep 16-byte alignment");
};
constexpr int kDk3KeysPerWg = 32 * kDkWaves;

template <int D, int MASK>
__global__ __launch_bounds__(kDkWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv3_kernel(BwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK >= 2;  // left bound in use (every wl_ test is guarded by it)
    constexpr bool SPARSE = MASK == 3;  // block map p.bmask with the window
    const int wl_ = MASK >= 2 ? p.wl : kUnbounded;
    const int wr_ = MASK >= 2 ? p.wr : 0;
    using QL = typename Dk3Lds<D>::QL;
    constexpr int TB = Dk3Lds<D>::TILE_BYTES;
    constexpr int SB = Dk3Lds<D>::STAGE_BYTES;
    constexpr int NST = kDk3Stages;
    constexpr int BQ = kDkBQ;
    constexpr int NC = D / 16;   // contraction steps of S and dP
    constexpr int NDB = D / 32;  // 32-dim blocks of dK and dV
    constexpr int PPW = QL::PIECES / kDkWaves;
    static_assert(QL::PIECES % kDkWaves == 0, "pieces must split over the waves");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;
    // unit = (batch, kv head, slice of its group's query heads)
    const int S = p.hsplit, Hs = p.Hkv * S;
    const int units = p.B * Hs;
    const int slot = blockIdx.x / units;
    const int unit = order_unit(blockIdx.x - slot * units, units, Hs, p.cu != nullptr);
    const int b = unit / Hs, gs = unit - (unit / Hs) * Hs;
    const int g = gs / S, sl = gs - (gs / S) * S;
    const int G = p.Hq / p.Hkv;
    const int GS = G / S;            // query heads of this workgroup
    const int h0 = g * G + sl * GS;  // the first of them
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    const int kstart = slot * kDk3KeysPerWg;
    if (kstart >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const int kw0 = kstart + 32 * w;  // first key of this wave (uniform)

    const size_t kvoff = sq.kvrow(g) * D;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;

    bf16x8 kreg[NC], vreg[NC];
    f32x16 dk[NDB], dv[NDB];
    {
        const int key = kw0 + l32;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            if (key < N) {
                kreg[cc] = as_bf16x8(ld16(Kh + size_t(key) * D + 16 * cc + 8 * hi));
                vreg[cc] = as_bf16x8(ld16(Vh + size_t(key) * D + 16 * cc + 8 * hi));
            } else {
                kreg[cc] = bf16x8{};
                vreg[cc] = bf16x8{};
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16{};
    }

    // Query tiles that can see a key of this workgroup (masked kernels: the
    // queries k - wr .. k + wl of each key k).
    const int nqt = (N + BQ - 1) / BQ;
    const int qt_first = CAUSAL ? max(0, kstart - wr_) / BQ : 0;
    const int qt_last = WIN ? min(nqt - 1, (kstart + kDk3KeysPerWg - 1 + wl_) / BQ) : nqt - 1;
    int per_head = qt_last - qt_first + 1;
    // Block-sparse: only the query tiles whose map block (row qt * 64 / 128,
    // column kstart / 128: one map column per workgroup) is visible, listed
    // in LDS after the stages.
    int* const tlist = reinterpret_cast<int*>(smem_raw + Dk3Lds<D>::BYTES);
    if constexpr (SPARSE) {
        const int col = kstart / kSparseBlock;
        if (w == 0) {
            const int cnt = compact_tiles(tlist, per_head, lane, [&](int t) {
                return int(p.bmask[size_t((qt_first + t) * BQ / kSparseBlock) * p.nb + col] != 0);
            });
            if (lane == 0) tlist[kSparseListCap] = cnt;
        }
        __syncthreads();
        per_head = __builtin_amdgcn_readfirstlane(lds_i32(tlist + kSparseListCap));
    }
    const int iters = GS * per_head;  // >= 1 unless a block map hides every query tile
    if (SPARSE && iters == 0) {
        // no query sees these keys: their gradients are zero
        bf16* dKh = static_cast<bf16*>(p.dK) + kvoff;
        bf16* dVh = static_cast<bf16*>(p.dV) + kvoff;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int kk = kw0 + 8 * (r >> 2) + 4 * hi + (r & 3);
                if (kk < N) {
                    const size_t e = size_t(kk) * D + db * 32 + l32;
                    if (S == 1) {
                        dKh[e] = bf16(0.f);
                        dVh[e] = bf16(0.f);
                    } else {
                        p.dk_part[sl * p.part_stride + kvoff + e] = 0.f;
                        p.dv_part[sl * p.part_stride + kvoff + e] = 0.f;
                    }
                }
            }
        return;
    }

    int src_off[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        int r, e0;
        QL::piece_src(w + kDkWaves * i, lane, r, e0);
        src_off[i] = r * D + e0;
    }
    auto tile_q0 = [&](int t) {
        if constexpr (SPARSE)
            return (qt_first + (__builtin_amdgcn_readfirstlane(lds_i32(tlist + t % per_head)) & 0xFFFFFF)) * BQ;
        else return (qt_first + t % per_head) * BQ;
    };
    // Copy of tile t into its stage by this wave, in 2 PPW + 1 pieces: piece
    // k < PPW is a 1 KB piece of Q, k < 2 PPW of dO, and piece 2 PPW the
    // tile's LSE and D (waves 0 and 1, 16 lanes).
    struct TileCopy {
        __amdgpu_buffer_rsrc_t q, o, stat;
        unsigned char* st;
        int last_row;  // rows past N read row N-1 (their results are hidden)
    };
    auto tile_copy = [&](int t) {
        const int hq = h0 + t / per_head;
        const int q0 = tile_q0(t);
        const size_t row0 = sq.qrow(hq) + q0;
        const uint32_t bytes = uint32_t(N - q0) * uint32_t(D * 2);
        TileCopy tc;
        tc.q = make_rsrc(static_cast<const bf16*>(p.Q) + row0 * D, bytes);
        tc.o = make_rsrc(static_cast<const bf16*>(p.dO) + row0 * D, bytes);
        tc.stat = make_rsrc((w == 0 ? p.LSE : p.Drow) + row0, uint32_t(N - q0) * 4u);
        tc.st = smem_raw + (t % NST) * SB;
        tc.last_row = N - 1 - q0;
        return tc;
    };
    auto copy_piece = [&](const TileCopy& tc, int k) {
        if (k < 2 * PPW) {
            const int i = k % PPW, pi = w + kDkWaves * i;
            const int r = src_off[i] / D;
            const uint32_t off = uint32_t(r <= tc.last_row ? src_off[i] : tc.last_row * D + src_off[i] % D);
            if (k < PPW) buf16_to_lds(tc.q, 2 * off, tc.st + 2 * QL::piece_dst(pi));
            else buf16_to_lds(tc.o, 2 * off, tc.st + TB + 2 * QL::piece_dst(pi));
        } else if (w < 2 && lane < 16) {
            buf16_to_lds(tc.stat, uint32_t(16 * lane), tc.st + 2 * TB + w * BQ * 4);
        }
    };
    auto issue = [&](int t) {
        const TileCopy tc = tile_copy(t);
#pragma unroll
        for (int k = 0; k <= 2 * PPW; ++k) copy_piece(tc, k);
    };
    // s_waitcnt vmcnt(n): n = this wave's copies of one tile (the newest tile stays in flight).
    auto wait_all_but_one_tile = [&]() {
        if (w < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PPW + 1) & 15) | (((2 * PPW + 1) >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PPW) & 15) | (((2 * PPW) >> 4) << 14));
    };

    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // Pipeline registers.  Every LDS read has one full step of slack: the
    // row fragments of A(i+2) are read during C(i), the transposed
    // fragments of C(i) and nothing else during A(i+1).
    bf16x8 aq[NC], ao[NC];          // row fragments of Q, dO: A operands of S, dP
    f32x4 lq4[4], dd4[4];           // LSE and D of the next B step's rows, in groups of 4
    f32x16 s0, dp0, s1, dp1;        // S, dP of two consecutive subtiles
    bf16x8 bo[2][NDB], bq[2][NDB];  // transposed dO, Q fragments of the current C step
    bf16x8 pb[2], sb[2];            // P^T, dS^T of the current subtile
    float pr[16], ds[16];

    auto stage = [&](int i) -> const unsigned char* { return smem_raw + ((i >> 1) % NST) * SB; };
    auto load_a = [&](int i, int cc) {
        const unsigned char* st = stage(i);
        const bf16* Qs = reinterpret_cast<const bf16*>(st) + 512 * (i & 1);
        const bf16* dOs = reinterpret_cast<const bf16*>(st + TB) + 512 * (i & 1);
        aq[cc] = as_bf16x8(lds16(Qs + QL::off(l32, 16 * cc + 8 * hi)));
        ao[cc] = as_bf16x8(lds16(dOs + QL::off(l32, 16 * cc + 8 * hi)));
    };
    auto load_stats = [&](int i, int j) {
        const float* ls = reinterpret_cast<const float*>(stage(i) + 2 * TB) + 32 * (i & 1);
        lq4[j] = lds_f32x4(ls + 8 * j + 4 * hi);
        dd4[j] = lds_f32x4(ls + BQ + 8 * j + 4 * hi);
    };
    // Transposing read number n (0 .. 8 NDB - 1) of subtile i's C step.
    auto load_tr = [&](int i, int n) {
        const unsigned char* st = stage(i);
        const int half = n & 1, which = (n >> 1) & 1, db = (n >> 2) % NDB, cc = (n >> 2) / NDB;
        const bf16* base = reinterpret_cast<const bf16*>(which ? st : st + TB);
        const int qr = 32 * (i & 1) + 16 * cc + trow + 8 * half;
        const bf16x4 v = lds_read_tr(base + QL::off(qr, db * 32 + tcol));
        bf16x8& dst = which ? bq[cc][db] : bo[cc][db];
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * half + e] = v[e];
    };
    auto needs_mask = [&](int i) {
        const int qb0 = tile_q0(i >> 1) + 32 * (i & 1);
        return (CAUSAL && (qb0 < kw0 + 31 - wr_ || (WIN && qb0 + 31 > kw0 + wl_))) || qb0 + 31 >= N;
    };
    constexpr int RPC = 16 / NC;       // score rows (registers) of B per slot
    constexpr int TPC = 8 * NDB / NC;  // transposing reads per slot
    static_assert(RPC * NC == 16 && TPC * NC == 8 * NDB && 2 * NDB == NC, "slots must divide the work");

    // Step 1 of subtile i, NC slots of two MFMAs: A(i+1), with B(i) (RPC
    // rows per slot) and the transposing reads of C(i).  Scheduling fences
    // keep the slots in order; the order inside a slot is the compiler's.
    auto step1 = [&](int i, const f32x16& s_cur, const f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt,
                     bool has_next, auto masked) {
        const int qb0 = tile_q0(i >> 1) + 32 * (i & 1);
        const int thr = CAUSAL ? kw0 + l32 - wr_ - qb0 - 4 * hi : -1 - 4 * hi;     // q < key - wr
        const int thr_hi = WIN ? kw0 + l32 + wl_ - qb0 - 4 * hi : kUnbounded;  // q > key + wl
        const int nlim = N - qb0 - 4 * hi;                                          // q >= N
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            if (has_next) {
                // the first product starts from an immediate zero (no register clearing)
                s_nxt = mfma_32x32x16(aq[k], kreg[k], k == 0 ? f32x16{} : s_nxt);
                dp_nxt = mfma_32x32x16(ao[k], vreg[k], k == 0 ? f32x16{} : dp_nxt);
            }
#pragma unroll
            for (int n = k * TPC; n < (k + 1) * TPC; ++n) load_tr(i, n);
#pragma unroll
            for (int r = k * RPC; r < (k + 1) * RPC; ++r) {
                float ex = fmaf(s_cur[r], c, -lq4[r >> 2][r & 3] * kLog2e);
                if constexpr (decltype(masked)::value) {
                    const int qo = 8 * (r >> 2) + (r & 3);
                    ex = (qo < thr || qo > thr_hi || qo >= nlim) ? -INFINITY : ex;
                }
                pr[r] = fast_exp2(ex);
                ds[r] = pr[r] * (dp_cur[r] - dd4[r >> 2][r & 3]);
                if ((r & 7) == 7) {
                    const int cc = r >> 3;
                    pb[cc] = to_bf16x8(pr[8 * cc + 0], pr[8 * cc + 1], pr[8 * cc + 2], pr[8 * cc + 3],
                                       pr[8 * cc + 4], pr[8 * cc + 5], pr[8 * cc + 6], pr[8 * cc + 7]);

                    sb[cc] = to_bf16x8(ds[8 * cc + 0], ds[8 * cc + 1], ds[8 * cc + 2], ds[8 * cc + 3],
                                       ds[8 * cc + 4], ds[8 * cc + 5], ds[8 * cc + 6], ds[8 * cc + 7]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Step 2 of subtile i, NC slots of two MFMAs: C(i), with the row reads of
    // A(i+2) and the statistics of subtile i+1.
    // Optionally also spreads the copy of a tile over the slots (one piece
    // per slot instead of a burst that queues in the address unit).
    auto step2 = [&](int i, bool has_next, bool has_next2) {
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const int cc = m / NDB, db = m % NDB;
            dv[db] = mfma_32x32x16(bo[cc][db], pb[cc], dv[db]);
            dk[db] = mfma_32x32x16(bq[cc][db], sb[cc], dk[db]);
            if (has_next2) load_a(i + 2, m);
            if (has_next && m < 4) load_stats(i + 1, m);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto body = [&](int i, const f32x16& s_cur, const f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, bool has_next,
                    bool has_next2) {
        __builtin_amdgcn_sched_barrier(0);
        if (needs_mask(i)) step1(i, s_cur, dp_cur, s_nxt, dp_nxt, has_next, std::true_type{});
        else step1(i, s_cur, dp_cur, s_nxt, dp_nxt, has_next, std::false_type{});
        if ((i & 1) == 0) {
            // Publish tile t+1: this wave's copies of it are done once only
            // tile t+2's remain in flight.  Tile t-1 was last read (and
            // waited for) in the previous body, so its stage is refilled
            // with tile t+3 right after the barrier.
            const int t = i >> 1;
            if (t + 2 < iters) wait_all_but_one_tile();
            else wait_vmem();
            __builtin_amdgcn_s_barrier();
            // One burst per wave: the address unit takes ~16 cycles per 1 KB
            // piece whichever way the pieces are spread over the step.
            if (t + 3 < iters) issue(t + 3);
        }
        __builtin_amdgcn_sched_barrier(0);
        step2(i, has_next, has_next2);
    };

    issue(0);
    if (iters > 1) issue(1);
    if (iters > 2) issue(2);
    if (iters > 2) {
        if (w < 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * PPW + 2) & 15) | (((4 * PPW + 2) >> 4) << 14));
        else __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * PPW) & 15) | (((4 * PPW) >> 4) << 14));
    } else if (iters > 1) {
        wait_all_but_one_tile();
    } else {
        wait_vmem();
    }
    __builtin_amdgcn_s_barrier();
    // A(0) outright, then the row reads of A(1) and the statistics of subtile 0.
    s0 = dp0 = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
        load_a(0, cc);
        s0 = mfma_32x32x16(aq[cc], kreg[cc], s0);
        dp0 = mfma_32x32x16(ao[cc], vreg[cc], dp0);
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) load_a(1, cc);
#pragma unroll
    for (int j = 0; j < 4; ++j) load_stats(0, j);

    const int nsub = 2 * iters;
    for (int i = 0; i + 2 < nsub; i += 2) {
        body(i, s0, dp0, s1, dp1, true, true);
        body(i + 1, s1, dp1, s0, dp0, true, true);
    }
    body(nsub - 2, s0, dp0, s1, dp1, true, false);
    body(nsub - 1, s1, dp1, s0, dp0, false, false);
    wait_vmem();  // no copy into LDS may outlive the workgroup

    // dK, dV (lane = key kw0 + l32, registers = dims): whole rows through
    // this wave's LDS region once every wave is past its last read.
    static_assert(kDkWaves * staged_rows_bytes<D, float>() <= int(Dk3Lds<D>::BYTES), "staging must fit");
    __syncthreads();
    unsigned char* stg = smem_raw + w * staged_rows_bytes<D, float>();
    const size_t row0 = kvoff + size_t(kw0) * D;
    if (S == 1) {
        store_rows_staged<D>(stg, dk, p.scale, static_cast<bf16*>(p.dK) + row0, N - kw0, lane);
        store_rows_staged<D>(stg, dv, 1.f, static_cast<bf16*>(p.dV) + row0, N - kw0, lane);
    } else {
        store_rows_staged<D>(stg, dk, p.scale, p.dk_part + sl * p.part_stride + row0, N - kw0, lane);
        store_rows_staged<D>(stg, dv, 1.f, p.dv_part + sl * p.part_stride + row0, N - kw0, lane);
    }
}

// ---------------------------------------------------------------- bwd_dq v2
// One workgroup of 8 waves per (batch, query head, 256 queries); each wave
// owns kDqRB 32-row blocks (Q and dO rows as B operands, dQ accumulators).
// With one block per wave (about 230 registers at d = 128) two waves share
// each SIMD, and one wave's softmax and dS arithmetic runs while the other's
// matrix products do (4 waves of two blocks each, which read every K / V
// fragment once for two products, measured 2-7 % slower).  K/V tiles of 64
// keys (padded K slabs: row reads for S^T = K Q^T, transposing reads for
// dQ^T += K^T dS^T) are copied global -> LDS by buffer loads, four stages
// with three tiles in flight (three stages measured 1 % slower).
constexpr int kDqRB = 1;  // 32-row blocks per wave
constexpr int kDqWaves = 8 / kDqRB;
constexpr int kDqBM = 256;
constexpr int kDqBN = 64;
constexpr int kDqStages = 4;

template <int D>
struct DqLds {
    using KL = PadSlab<kDqBN, D>;
    static constexpr int TILE_BYTES = KL::ELEMS * 2;
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
    static constexpr size_t BYTES = size_t(kDqStages) * STAGE_BYTES;
};

template <int D, int MASK, bool DROP>
__global__ __launch_bounds__(kDqWaves * 64) __attribute__((amdgpu_waves_per_eu(kDqWaves / 4, kDqWaves / 4)))
void bwd_dq2_kernel(BwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK >= 2;  // left bound in use (every wl_ test is guarded by it)
    constexpr bool SPARSE = MASK == 3;  // block map p.bmask with the window
    const int wl_ = MASK >= 2 ? p.wl : kUnbounded;
    const int wr_ = MASK >= 2 ? p.wr : 0;
    using KL = typename DqLds<D>::KL;
    constexpr int TB = DqLds<D>::TILE_BYTES;
    constexpr int SB = DqLds<D>::STAGE_BYTES;
    constexpr int NST = kDqStages;
    constexpr int BN = kDqBN;
    constexpr int PPW = KL::PIECES / kDqWaves;
    static_assert(KL::PIECES % kDqWaves == 0, "pieces must split over the waves");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem_raw[];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const float c = p.scale_log2;
    const int units = p.B * p.Hq;
    const int slot = blockIdx.x / units;
    const int unit = order_unit(blockIdx.x - slot * units, units, p.Hq, p.cu != nullptr);
    const int qb = CAUSAL ? p.nqb - 1 - slot : slot;
    const int b = unit / p.Hq, h = unit - (unit / p.Hq) * p.Hq;
    const int g = h / (p.Hq / p.Hkv);
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    if (qb * kDqBM >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const size_t qrows = sq.qrow(h);
    const size_t kvoff = sq.kvrow(g) * D;
    const bf16* __restrict__ Qh = static_cast<const bf16*>(p.Q) + qrows * D;
    const bf16* __restrict__ dOh = static_cast<const bf16*>(p.dO) + qrows * D;
    const bf16* __restrict__ Kh = static_cast<const bf16*>(p.K) + kvoff;
    const bf16* __restrict__ Vh = static_cast<const bf16*>(p.V) + kvoff;

    const int q0 = qb * kDqBM;
    constexpr int RB = kDqRB;
    const int wq0 = q0 + 32 * RB * w;
    const int wq_last = wq0 + 32 * RB - 1;

    bf16x8 qreg[RB][D / 16], oreg[RB][D / 16];
    float lse2[RB], drow[RB];
    int key_lim[RB], key_lo[RB];  // visible keys of each row block's lane: key_lo .. key_lim
    f32x16 acc[RB][D / 32];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int qrow = wq0 + 32 * rb + l32;
#pragma unroll
        for (int cc = 0; cc < D / 16; ++cc) {
            if (qrow < N) {
                qreg[rb][cc] = as_bf16x8(ld16(Qh + size_t(qrow) * D + 16 * cc + 8 * hi));
                oreg[rb][cc] = as_bf16x8(ld16(dOh + size_t(qrow) * D + 16 * cc + 8 * hi));
            } else {
                qreg[rb][cc] = bf16x8{};
                oreg[rb][cc] = bf16x8{};
            }
        }
        // rows past N: LSE = +inf makes P exactly 0
        lse2[rb] = (qrow < N) ? p.LSE[qrows + qrow] * kLog2e : INFINITY;
        drow[rb] = (qrow < N) ? p.Drow[qrows + qrow] : 0.f;
        key_lim[rb] = CAUSAL ? min(qrow + wr_, N - 1) : N - 1;
        key_lo[rb] = WIN ? qrow - wl_ : 0;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[rb][db] = f32x16{};
    }

    // Key tiles [kt0, kt0 + ntiles): masked kernels see keys q - wl .. q + wr.
    const int kend = CAUSAL ? min(N, q0 + kDqBM + wr_) : N;
    const int kt0 = WIN ? max(0, q0 - wl_) / BN : 0;
    int ntiles = (kend + BN - 1) / BN - kt0;
    // Block-sparse: the key tiles whose map block is visible to the rows of
    // waves 0-1 (map row q0 / 128, tag bit 0) or waves 2-3 (the next row,
    // bit 1), listed in LDS after the stages.
    int* const tlist = reinterpret_cast<int*>(smem_raw + DqLds<D>::BYTES);
    if constexpr (SPARSE) {
        const int r0 = q0 / kSparseBlock;
        if (w == 0) {
            const int cnt = compact_tiles(tlist, ntiles, lane, [&](int t) {
                const int col = (kt0 + t) * BN / kSparseBlock;
                return int(p.bmask[size_t(r0) * p.nb + col] != 0) |
                       (r0 + 1 < p.nb && p.bmask[size_t(r0 + 1) * p.nb + col] != 0 ? 2 : 0);
            });
            if (lane == 0) tlist[kSparseListCap] = cnt;
        }
        __syncthreads();
        ntiles = __builtin_amdgcn_readfirstlane(lds_i32(tlist + kSparseListCap));
    }
    auto tile_key0 = [&](int kt) -> int {
        if constexpr (SPARSE) return (kt0 + (__builtin_amdgcn_readfirstlane(lds_i32(tlist + kt)) & 0xFFFFFF)) * BN;
        else return (kt0 + kt) * BN;
    };
    auto wave_sees = [&](int kt) -> bool {
        if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(lds_i32(tlist + kt)) >> (24 + (wq0 - q0) / 128)) & 1;
        else return true;
    };

    int src_off[PPW];
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        int r, e0;
        KL::piece_src(w + kDqWaves * i, lane, r, e0);
        src_off[i] = r * D + e0;
    }
    auto issue = [&](int kt) {
        const int key0 = tile_key0(kt);
        unsigned char* st = smem_raw + (kt % NST) * SB;
        const uint32_t bytes = uint32_t(N - key0) * uint32_t(D * 2);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(Kh + size_t(key0) * D, bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vh + size_t(key0) * D, bytes);
        const bool tail = key0 + BN > N;
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
            const int pi = w + kDqWaves * i;
            uint32_t off = uint32_t(src_off[i]);
            if (tail) off = uint32_t(min(src_off[i] / D, N - 1 - key0) * D + src_off[i] % D);
            buf16_to_lds(kr, 2 * off, st + 2 * KL::piece_dst(pi));
            buf16_to_lds(vr, 2 * off, st + TB + 2 * KL::piece_dst(pi));
        }
    };

    const int trow = 4 * hi + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    if (ntiles > 0) issue(0);
    if (ntiles > 1) issue(1);
    if (ntiles > 2) issue(2);
    wait_vmem();
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        if (kt + 3 < ntiles) issue(kt + 3);
        const bf16* Ks = reinterpret_cast<const bf16*>(smem_raw + (kt % NST) * SB);
        const bf16* Vs = reinterpret_cast<const bf16*>(smem_raw + (kt % NST) * SB + TB);
        const int kstart = tile_key0(kt);
        const bool sees = wave_sees(kt);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
            const int kb0 = kstart + 32 * kb;
            if (!sees || (CAUSAL && (kb0 > wq_last + wr_ || (WIN && kb0 + 31 < wq0 - wl_))) || kb0 >= N) continue;
            // S^T = K Q^T, dP^T = V dO^T for both row blocks: lane = query,
            // register r = key kb0 + 8(r/4) + 4hi + r%4
            f32x16 s[RB], dpt[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) s[rb] = dpt[rb] = f32x16{};
#pragma unroll
            for (int cc = 0; cc < D / 16; ++cc) {
                const bf16x8 ak = as_bf16x8(lds16(Ks + KL::off(32 * kb + l32, 16 * cc + 8 * hi)));
                const bf16x8 av = as_bf16x8(lds16(Vs + KL::off(32 * kb + l32, 16 * cc + 8 * hi)));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    s[rb] = mfma_32x32x16(ak, qreg[rb][cc], s[rb]);
                    dpt[rb] = mfma_32x32x16(av, oreg[rb][cc], dpt[rb]);
                }
            }
            bf16x8 sb[RB][2];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                float ds[16];
                uint32_t dy[4];  // dropout keep bytes: dP is dropped and scaled before dS
                if constexpr (DROP)
                    drop_bytes_qmajor(dy, wq0 + 32 * rb + l32, kb0, hi, lane, uint32_t(b * p.Hq + h), p.drop_off,
                                      p.drop_k0, p.drop_k1);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float pr = fast_exp2(fmaf(s[rb][r], c, -lse2[rb]));
                    if constexpr (DROP) {
                        const float dpd = drop_keep(dy, r, p.drop_t8) ? dpt[rb][r] * (256.f / float(256 - p.drop_t8))
                                                                       : 0.f;
                        ds[r] = pr * (dpd - drow[rb]);
                    } else {
                        ds[r] = pr * (dpt[rb][r] - drow[rb]);
                    }
                }
                if ((CAUSAL && (kb0 + 31 > wq0 + 32 * rb + wr_ || (WIN && kb0 < wq0 + 32 * rb + 31 - wl_))) ||
                    kb0 + 31 >= N) {
                    const int lim = key_lim[rb] - kb0 - 4 * hi;
                    const int lo = key_lo[rb] - kb0 - 4 * hi;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = 8 * (r >> 2) + (r & 3);
                        ds[r] = (kk > lim || (WIN && kk < lo)) ? 0.f : ds[r];
                    }
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc)
                    sb[rb][cc] = to_bf16x8(ds[8 * cc + 0], ds[8 * cc + 1], ds[8 * cc + 2], ds[8 * cc + 3], ds[8 * cc + 4],
                                           ds[8 * cc + 5], ds[8 * cc + 6], ds[8 * cc + 7]);
            }
            // dQ^T += K^T dS^T: K^T through transposing reads, each fragment feeding two products
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int kr = 32 * kb + 16 * cc + trow;
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const bf16x8 a = cat(lds_read_tr(Ks + KL::off(kr, db * 32 + tcol)),
                                         lds_read_tr(Ks + KL::off(kr + 8, db * 32 + tcol)));
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) acc[rb][db] = mfma_32x32x16(a, sb[rb][cc], acc[rb][db]);
                }
            }
        }
        // as in the dK/dV kernel: own copies of the next tile, LDS reads
        // drained, plain barrier (no fence waiting for the newer copies)
        const int ahead = min(ntiles - 1, kt + 3) - (kt + 1);  // tiles issued after kt + 1
        if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | ((4 * PPW) & 15) | (((4 * PPW) >> 4) << 14));
        else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * PPW) & 15) | (((2 * PPW) >> 4) << 14));
        else wait_vmem();
        barrier_lds();
    }

    // dQ (lane = query row): whole rows through this wave's LDS region once
    // every wave is past its last read.
    static_assert(kDqWaves * staged_rows_bytes<D, bf16>() <= int(DqLds<D>::BYTES), "staging must fit");
    __syncthreads();
    unsigned char* stg = smem_raw + w * staged_rows_bytes<D, bf16>();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int r0 = wq0 + 32 * rb;
        store_rows_staged<D>(stg, acc[rb], p.scale, static_cast<bf16*>(p.dQ) + qrows * D + size_t(r0) * D, N - r0, lane);
    }
}

template <int D, int MASK, bool DROP = false>
hipError_t launch_bwd_t(BwdParams p, hipStream_t stream) {
    // 1. D_i = dO_i . O_i
    // Every query row of every head: [B, Hq, N] rows, or [Hq, total] packed.
    const long long rows = p.cu != nullptr ? (long long)p.Hq * p.total : (long long)p.B * p.Hq * p.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(unsigned((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                       static_cast<const bf16*>(p.O), static_cast<const bf16*>(p.dO), p.Drow, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. dK, dV
    constexpr size_t list_bytes = MASK == 3 ? size_t(kSparseListCap + 1) * sizeof(int) : 0;
    if constexpr ((D == 128 || MASK == 3) && !DROP) {
        auto kern = bwd_dkdv3_kernel<D, MASK>;
        constexpr size_t lds = Dk3Lds<D>::BYTES + list_bytes;
        static DeviceOnce attr;
        if ((e = set_max_dynamic_lds(kern, lds, attr)) != hipSuccess) return e;
        p.nkb = (p.N + kDk3KeysPerWg - 1) / kDk3KeysPerWg;
        const long long blocks = (long long)p.nkb * p.B * p.Hkv * p.hsplit;
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kDkWaves * 64), lds, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        auto kern = bwd_dkdv2_kernel<D, MASK, DROP>;
        constexpr size_t lds = DkLds<D>::BYTES;
        static DeviceOnce attr;
        if ((e = set_max_dynamic_lds(kern, lds, attr)) != hipSuccess) return e;
        p.nkb = (p.N + dk_keys_per_wg<D>() - 1) / dk_keys_per_wg<D>();
        const long long blocks = (long long)p.nkb * p.B * p.Hkv * p.hsplit;
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(DkCfg<D>::NW * 64), lds, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 2b. sum of the query-head slices' partials
    if (p.hsplit > 1) {
        const long long n4 = (long long)p.B * p.Hkv * p.N * D / 4;
        hipLaunchKernelGGL(dkdv_reduce_kernel, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, stream, p.dk_part,
                           p.dv_part, static_cast<bf16*>(p.dK), static_cast<bf16*>(p.dV), n4, p.hsplit,
                           p.part_stride);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // 3. dQ
    {
        auto kern = bwd_dq2_kernel<D, MASK, DROP>;
        constexpr size_t lds = DqLds<D>::BYTES + list_bytes;
        static DeviceOnce attr;
        if ((e = set_max_dynamic_lds(kern, lds, attr)) != hipSuccess) return e;
        p.nqb = (p.N + kDqBM - 1) / kDqBM;
        const long long blocks = (long long)p.nqb * p.B * p.Hq;
        hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kDqWaves * 64), lds, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_bf16(BwdParams p, int d, int causal, hipStream_t stream) {
    // 0: no mask, 1: causal, 2: a general window, 3: block map (and window)
    const int mk = p.bmask != nullptr ? 3 : !causal ? 0 : (p.wl >= kUnbounded && p.wr == 0) ? 1 : 2;
    if (p.drop_t8 > 0) {
        // dropout: fixed-length batches, no window or map (the entry point checks)
        if (d == 64) return mk == 0 ? launch_bwd_t<64, 0, true>(p, stream) : launch_bwd_t<64, 1, true>(p, stream);
        if (d == 128) return mk == 0 ? launch_bwd_t<128, 0, true>(p, stream) : launch_bwd_t<128, 1, true>(p, stream);
        return hipErrorNotSupported;
    }
    switch (d) {
        case 64:
            return mk == 0   ? launch_bwd_t<64, 0>(p, stream)
                   : mk == 1 ? launch_bwd_t<64, 1>(p, stream)
                   : mk == 2 ? launch_bwd_t<64, 2>(p, stream)
                             : launch_bwd_t<64, 3>(p, stream);
        case 128:
            return mk == 0   ? launch_bwd_t<128, 0>(p, stream)
                   : mk == 1 ? launch_bwd_t<128, 1>(p, stream)
                   : mk == 2 ? launch_bwd_t<128, 2>(p, stream)
                             : launch_bwd_t<128, 3>(p, stream);
        default: return hipErrorNotSupported;
    }
}

hipError_t launch_bwd_f32(BwdParams, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa
