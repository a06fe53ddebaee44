// Device-side building blocks for the gfx950 attention kernels.
//
// Matrix-core layouts (v_mfma_f32_32x32x16_bf16, one 64-lane wave; lane l,
// half h = l / 32):
//   A (32 x 16):  lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32):  lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32):  lane l, register r holds C[8(r/4) + 4h + r%4][l % 32]
// LDS transpose read (ds_read_b64_tr_b16), per group of 16 lanes: lanes
// 4e..4e+3 each address 4 consecutive 16-bit elements that together form
// row e (16 elements); lane i of the group receives column i of rows 0..3.
// v_permlane32_swap(x, x) returns {x[l % 32], x[32 + l % 32]} in every lane.
// These were checked on the device with a layout probe before use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Rows of one attention unit (batch entry or packed sequence b) in the
// query-side and key-side buffers.  Fixed-length batch ([B, H, N, d]): head h
// of entry b starts at row (b*H + h)*N and has N rows.  Packed sequences
// ([H, total, d] with offsets cu[0..B]): sequence b of head h starts at row
// h*total + cu[b] and has cu[b+1] - cu[b] rows.  The offsets are clamped
// into [0, total] and the length to at most N (the bound the grid was sized
// for), so every access stays inside the buffers whatever the offsets hold.
struct SeqSpan {
    size_t qbase, kvbase, hstride;
    int n;  // rows of this unit
    __device__ __forceinline__ size_t qrow(int h) const { return qbase + size_t(h) * hstride; }
    __device__ __forceinline__ size_t kvrow(int g) const { return kvbase + size_t(g) * hstride; }
};

__device__ __forceinline__ SeqSpan seq_span(const int* cu, int total, int Hq, int Hkv, int N, int b) {
    SeqSpan s;
    if (cu != nullptr) {
        const int a = min(max(cu[b], 0), total);
        const int e = min(max(cu[b + 1], a), total);
        s.qbase = s.kvbase = size_t(a);
        s.hstride = size_t(total);
        s.n = min(e - a, N);
    } else {
        s.qbase = size_t(b) * size_t(Hq) * size_t(N);
        s.kvbase = size_t(b) * size_t(Hkv) * size_t(N);
        s.hstride = size_t(N);
        s.n = N;
    }
    return s;
}

// Workgroup unit slot u (0 <= u < units = B*H; workgroups are dealt to the
// 8 XCDs round-robin, so u % 8 picks the XCD) -> unit b*H + h.
// Fixed-length batch (every unit costs the same): when units % 8 == 0,
// consecutive units go to one XCD so heads sharing K/V share its L2.
// Packed sequences (units of very different cost): every XCD takes the same
// slice of heads of every sequence -- heads [x*H/8, (x+1)*H/8) on XCD x when
// H % 8 == 0 (grouped query heads stay together when their group divides
// H/8), round-robin otherwise -- so no XCD gets a long sequence's heads alone.
__device__ __forceinline__ int order_unit(int u, int units, int H, bool packed) {
    if (packed) {
        if (H % 8 != 0) return u;
        const int hp = H >> 3, x = u & 7, j = u >> 3;
        const int b = j / hp;
        return b * H + x * hp + (j - b * hp);
    }
    return (units % 8 == 0) ? (u & 7) * (units >> 3) + (u >> 3) : u;
}

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte LDS / global vector access helpers.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

// LDS reads of data that arrives by direct buffer-to-LDS copies.  The
// restrict-qualified pointer gives each read scoped alias information; the
// compiler then leaves the wait for those copies (s_waitcnt vmcnt) to the
// kernel, which waits for its own copies explicitly before the barrier that
// publishes a tile, instead of waiting for every copy in flight (including
// prefetches of later tiles) before the first LDS read.
__device__ __forceinline__ u32x4 lds16(const void* __restrict__ p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ f32x4 lds_f32x4(const float* __restrict__ p) {
    return *reinterpret_cast<const f32x4*>(p);
}

__device__ __forceinline__ int lds_i32(const int* __restrict__ p) { return *p; }

// Compacts, within one wave, the indices t in [0, n) whose tag(t) is
// nonzero into list[0 .. count) in ascending order, each stored as
// t | tag(t) << 24 (t < 2^24, tag < 128); returns count (wave-uniform).
template <typename F>
__device__ __forceinline__ int compact_tiles(int* list, int n, int lane, F tag) {
    int count = 0;
    for (int base = 0; base < n; base += 64) {
        const int t = base + lane;
        const int tg = t < n ? tag(t) : 0;
        const unsigned long long bal = __ballot(tg != 0);
        if (tg != 0) {
            const int below = __builtin_amdgcn_mbcnt_hi(uint32_t(bal >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0));
            list[count + below] = t | (tg << 24);
        }
        count += __popcll(bal);
    }
    return count;
}

// ---------------------------------------------------------------------------
// Dropout bits.  Philox-4x32 with 10 rounds (J. K. Salmon, M. A. Moraes,
// R. O. Dror, D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
// SC 2011): per round the counter words 0 and 2 are multiplied (full 64-bit
// products) by 0xD2511F53 and 0xCD9E8D57, the new counter is
// (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), and the key is bumped by
// (0x9E3779B9, 0xBB67AE85) between rounds.
// One call gives the 16 keep bytes of a 4 x 4 block of (query, key):
// counter (key / 4, query / 4, batch * H_q + head, offset), word q % 4 is
// the block's query row, byte k % 4 of it the key.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = uint64_t(0xD2511F53u) * c0;
        const uint64_t p1 = uint64_t(0xCD9E8D57u) * c2;
        c0 = uint32_t(p1 >> 32) ^ c1 ^ k0;
        c1 = uint32_t(p1);
        c2 = uint32_t(p0 >> 32) ^ c3 ^ k1;
        c3 = uint32_t(p0);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return u32x4{c0, c1, c2, c3};
}

// In every group of 4 lanes (l % 4 = s), lane s ends with x[g] = the input
// x[s] of lane g: a 4 x 4 transpose of words over the lane quad, in two
// exchanges with the lanes s ^ 2 and s ^ 1 (DPP quad permutations).
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int lane) {
    const bool b1 = (lane & 2) != 0, b0 = (lane & 1) != 0;
    {
        const uint32_t s0 = b1 ? x[0] : x[2], s1 = b1 ? x[1] : x[3];
        const uint32_t r0 = uint32_t(__builtin_amdgcn_mov_dpp(int(s0), 0x4E, 0xF, 0xF, false));  // lanes [2,3,0,1]
        const uint32_t r1 = uint32_t(__builtin_amdgcn_mov_dpp(int(s1), 0x4E, 0xF, 0xF, false));
        if (b1) {
            x[0] = r0;
            x[1] = r1;
        } else {
            x[2] = r0;
            x[3] = r1;
        }
    }
    {
        const uint32_t s0 = b0 ? x[0] : x[1], s1 = b0 ? x[2] : x[3];
        const uint32_t r0 = uint32_t(__builtin_amdgcn_mov_dpp(int(s0), 0xB1, 0xF, 0xF, false));  // lanes [1,0,3,2]
        const uint32_t r1 = uint32_t(__builtin_amdgcn_mov_dpp(int(s1), 0xB1, 0xF, 0xF, false));
        if (b0) {
            x[0] = r0;
            x[2] = r1;
        } else {
            x[1] = r0;
            x[3] = r1;
        }
    }
}

// Keep bytes for the score layout with one query per lane (S^T = K Q^T:
// lane query `q`, register r = key kb0 + 8 (r / 4) + 4 hi + r % 4, kb0 a
// multiple of 32, the lane quad holding queries 4 (q / 4) .. +3): on return
// byte t of y[g] is the byte of (q, kb0 + 8 g + 4 hi + t).  Each lane of a
// quad draws one key group's block, the quad transpose hands every lane its
// own query row of all four.
__device__ __forceinline__ void drop_bytes_qmajor(uint32_t (&y)[4], int q, int kb0, int hi, int lane, uint32_t bh,
                                                  uint32_t off, uint32_t k0, uint32_t k1) {
    const int s = lane & 3;
    const u32x4 w = philox4x32_10(uint32_t(kb0 + 8 * s + 4 * hi) >> 2, uint32_t(q) >> 2, bh, off, k0, k1);
    y[0] = w[0];
    y[1] = w[1];
    y[2] = w[2];
    y[3] = w[3];
    quad_transpose(y, lane);
}

// Keep bytes for the score layout with one key per lane (S = Q K^T: lane
// key `k`, register r = query qb0 + 8 (r / 4) + 4 hi + r % 4, qb0 a multiple
// of 32, the lane quad holding keys 4 (k / 4) .. +3): on return byte t of
// y[g] is the byte of (qb0 + 8 g + 4 hi + t, k).  Each lane draws one query
// group's block, regroups its bytes by key (byte d of word t -> byte t of
// word d, v_perm), and the quad transpose hands every lane its key's bytes.
__device__ __forceinline__ void drop_bytes_kmajor(uint32_t (&y)[4], int k, int qb0, int hi, int lane, uint32_t bh,
                                                  uint32_t off, uint32_t k0, uint32_t k1) {
    const int s = lane & 3;
    const u32x4 w = philox4x32_10(uint32_t(k) >> 2, uint32_t(qb0 + 8 * s + 4 * hi) >> 2, bh, off, k0, k1);
    const uint32_t a_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // w0.b0 w1.b0 w0.b1 w1.b1
    const uint32_t a_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // w0.b2 w1.b2 w0.b3 w1.b3
    const uint32_t b_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t b_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    y[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);  // byte 0 of w0..w3
    y[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);  // byte 1
    y[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);  // byte 2
    y[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);  // byte 3
    quad_transpose(y, lane);
}

// Byte t of word y[g] >= the threshold: element r = 4 g + t is kept.
__device__ __forceinline__ bool drop_keep(const uint32_t (&y)[4], int r, int t8) {
    return int((y[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= t8;
}

// Transposing 8-byte LDS read (see the layout note at the top).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* __restrict__ p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
#pragma clang diagnostic pop
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Max of x over lanes l and l^32 (the two halves of the wave).
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (int)r[0]), __builtin_bit_cast(float, (int)r[1]));
}
// Sum of x over lanes l and l^32.
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
    return __builtin_bit_cast(float, (int)r[0]) + __builtin_bit_cast(float, (int)r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even float -> bf16 pairs (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                            float a7) {
    return bf16x8{(bf16)a0, (bf16)a1, (bf16)a2, (bf16)a3, (bf16)a4, (bf16)a5, (bf16)a6, (bf16)a7};
}

// ---------------------------------------------------------------------------
// LDS tile layouts.  A tile is `rows` x D bf16 stored as 16-byte chunks with
// no padding; chunk c of row r lives at chunk slot r * (D/8) + swz(r, c).
// The XOR swizzles keep the gfx950 LDS (64 banks x 4 bytes = 16 chunk slots
// per bank row) free of conflicts for the access patterns that use them:
//
//  row-read layout (ds_read_b128 of one chunk from 16 consecutive rows):
//    D >= 128: c ^ (r % 16)     D == 64: c ^ ((r / 2) % 8)
//  transpose-read layout (ds_read_b64_tr_b16 of 4 chunks from 4 rows,
//  rows r0..r0+3 with r0 % 4 == 0, chunks 4k..4k+3):
//    D >= 128: c ^ 4(r % 4)     D == 64: c ^ 4((r / 2) % 2)
// Writing whole rows (16 lanes = 16 consecutive chunks) is conflict-free in
// both layouts.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz_row(int r, int c) {
    if constexpr (D >= 128) return c ^ (r & 15);
    else return c ^ ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_tr(int r, int c) {
    if constexpr (D >= 128) return c ^ ((r & 3) << 2);
    else return c ^ (((r >> 1) & 1) << 2);
}
// Layout read both ways (row reads of 16 rows r0..r0+15 with r0 % 16 == 0,
// and transpose reads of rows r0..r0+3 x chunks 4k..4k+3):
//    D >= 128: c ^ (4(r % 4) | (r / 4) % 4)
//    D == 64:  c ^ (4((r / 2) % 2) | (r / 4) % 4)
// Row reads: the XOR term is a bijection over the 16 rows (per row parity
// for D == 64), so one chunk column lands in 16 distinct slots.  Transpose
// reads: the (r % 4) bits move whole 4-chunk groups, the (r / 4) bits
// permute inside a group, giving 16 distinct slots for the 4 x 4 block.
template <int D>
__device__ __forceinline__ int swz_both(int r, int c) {
    if constexpr (D >= 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int off_both(int r, int e) {
    return r * D + (swz_both<D>(r, e >> 3) << 3) + (e & 7);
}
// Slab layouts (every fragment a fixed offset from one per-lane base, so LDS
// reads take immediate offsets instead of per-fragment address registers):
//  K slabs: a ROWS x D tile as D/16 slabs of ROWS x 16 elements; within a
//    32-byte row the two 16-byte halves are swapped when bit 3 of the row is
//    set, so 16 consecutive rows of one half land in 16 distinct bank slots.
//  V slabs: D/32 slabs of ROWS x 32 elements, rows of 64 bytes: a transpose
//    read of 4 rows x 64 bytes covers all 64 banks exactly once.
template <int ROWS>
__device__ __forceinline__ int kslab_off(int r, int e) {
    return (e >> 4) * ROWS * 16 + r * 16 + 8 * (((e >> 3) & 1) ^ ((r >> 3) & 1)) + (e & 7);
}
template <int ROWS>
__device__ __forceinline__ int vslab_off(int r, int e) {
    return (e >> 5) * ROWS * 32 + r * 32 + (e & 31);
}
// Inverse maps: 16-byte slot s of the tile -> (row, first element of the chunk).
template <int ROWS>
__device__ __forceinline__ void kslab_slot(int s, int& r, int& e0) {
    const int cc = s / (2 * ROWS), rem = s - cc * 2 * ROWS;
    r = rem >> 1;
    e0 = 16 * cc + 8 * ((rem & 1) ^ ((r >> 3) & 1));
}
template <int ROWS>
__device__ __forceinline__ void vslab_slot(int s, int& r, int& e0) {
    const int db = s / (4 * ROWS), rem = s - db * 4 * ROWS;
    r = rem >> 2;
    e0 = 32 * db + 8 * (rem & 3);
}
// Padded K slabs: K slabs with a 128-byte gap after every slab.  Serves both
// 16-byte row reads (MFMA A operands) and transposing reads (B operands of
// the transposed product) without bank conflicts: the gap puts the two
// 16-dim slabs touched by one transposing read in different bank halves.
template <int ROWS, int D>
struct PadSlab {
    static constexpr int SLAB = ROWS * 16 + 64;   // elements per slab incl. gap
    static constexpr int ELEMS = (D / 16) * SLAB;  // elements per tile
    static constexpr int PIECES_PER_SLAB = ROWS / 32;  // 1 KB copy pieces
    static constexpr int PIECES = (D / 16) * PIECES_PER_SLAB;
    static __device__ __forceinline__ int off(int r, int e) {
        return (e >> 4) * SLAB + r * 16 + 8 * (((e >> 3) & 1) ^ ((r >> 3) & 1)) + (e & 7);
    }
    // LDS element offset of the start of copy piece p.
    static __device__ __forceinline__ int piece_dst(int p) {
        return (p / PIECES_PER_SLAB) * SLAB + (p % PIECES_PER_SLAB) * 512;
    }
    // Source (row, first element) of the 16 bytes lane l of piece p copies.
    static __device__ __forceinline__ void piece_src(int p, int l, int& r, int& e0) {
        const int slab = p / PIECES_PER_SLAB, s = (p % PIECES_PER_SLAB) * 64 + l;
        r = s >> 1;
        e0 = 16 * slab + 8 * ((s & 1) ^ ((r >> 3) & 1));
    }
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Buffer resource over `bytes` bytes at `base` (raw buffer, gfx9 descriptor
// word 3 = 0x00020000).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 16-byte buffer load straight into LDS: lane l writes dst_uniform + 16 l.
__device__ __forceinline__ void buf16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* dst_uniform) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wold-style-cast"
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)dst_uniform, 16, voff, 0, 0, 0);
#pragma clang diagnostic pop
}
// Wait for this wave's outstanding vector-memory loads (including
// direct-to-LDS copies): s_waitcnt vmcnt(0), other counters at maximum.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait for this wave's outstanding LDS operations: s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier for kernels whose LDS tiles arrive by direct
// buffer-to-LDS copies.  Every wave has already waited for its own copies
// of the tile being published (s_waitcnt vmcnt); draining this wave's LDS
// reads first keeps a later copy into a reused stage from overtaking them.
// Unlike __syncthreads(), whose fence also waits for every copy still in
// flight (the prefetches of later tiles), this waits for nothing else.
__device__ __forceinline__ void barrier_lds() {
    wait_lds();
    __builtin_amdgcn_s_barrier();
}

// Stores 32 rows of a row-major [rows, D] matrix that one wave holds in the
// accumulator layout of 32x32x16 products with the row as the N index (lane
// l: row l % 32; register r of block db: column 32 db + 8 (r / 4) +
// 4 (l / 32) + r % 4), scaled by f and converted to T (bf16 or float).  The
// rows pass through the wave's own LDS region `stg` (32 (D sizeof(T) + 16)
// bytes, 16-byte aligned, free of every other wave's use) so that each
// global store writes whole rows, 16 bytes per lane, rather than four
// values per lane scattered over 64 rows.  Rows at or past `nrows` are
// skipped; LD is the row stride of dst in elements (D, or more when the
// call stores a column slice of wider rows).  LDS operations of one wave
// execute in order, so the region can be reused for the next matrix (or
// slice) straight away.
template <int D, typename T, int LD = D>
__device__ __forceinline__ void store_rows_staged(unsigned char* stg, const f32x16* acc, float f, T* dst, int nrows,
                                                  int lane) {
    constexpr int ES = int(sizeof(T));
    constexpr int ROWB = D * ES + 16;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            unsigned char* a = stg + l32 * ROWB + (db * 32 + 8 * g + 4 * hi) * ES;
            const float x0 = acc[db][4 * g] * f, x1 = acc[db][4 * g + 1] * f;
            const float x2 = acc[db][4 * g + 2] * f, x3 = acc[db][4 * g + 3] * f;
            if constexpr (ES == 2) *reinterpret_cast<bf16x4*>(a) = bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3};
            else *reinterpret_cast<f32x4*>(a) = f32x4{x0, x1, x2, x3};
        }
    constexpr int LPR = D * ES / 16;  // lanes per row
    constexpr int RPI = 64 / LPR;     // rows per read
    static_assert(LPR * RPI == 64 && 32 % RPI == 0, "rows must tile the wave");
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
        const int row = it * RPI + lane / LPR, c = lane % LPR;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + row * ROWB + c * 16);
        if (row < nrows) *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(dst + size_t(row) * LD) + c * 16) = v;
    }
}
template <int D, typename T>
constexpr int staged_rows_bytes() {
    return 32 * (D * int(sizeof(T)) + 16);
}

// Element offset of (row r, element e) in a row-read tile.
template <int D>
__device__ __forceinline__ int off_row(int r, int e) {
    return r * D + (swz_row<D>(r, e >> 3) << 3) + (e & 7);
}
template <int D>
__device__ __forceinline__ int off_tr(int r, int e) {
    return r * D + (swz_tr<D>(r, e >> 3) << 3) + (e & 7);
}

}  // namespace fa
