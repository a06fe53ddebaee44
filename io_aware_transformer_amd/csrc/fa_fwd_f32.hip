// Forward pass with float32 inputs and outputs, fp32 vector arithmetic.
//
// Same tile-by-tile online softmax as the bf16 kernel (FlashAttention
// interview Q&A, app.wittybyte.ai "FlashAttention1", softmax answer;
// output rescaling from the deep-dive page's "Intuition"), written for
// accuracy rather than speed: every product and sum is an fp32 FMA.  One
// workgroup of 4 waves per (batch, query head, 64 query rows); each row is
// served by 4 lanes that each own a quarter of the head dimension (float4
// groups interleaved so the 4 lanes read 64 consecutive bytes of a K/V row).
#include "fa_device.hpp"
#include "fa_internal.h"

#include <math.h>

namespace fa {

namespace {

constexpr int kBM32 = 64;  // query rows per workgroup
constexpr int kBN32 = 32;  // keys per tile

template <int D, int MASK>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
    // MASK 0: no mask; 1: causal (window (unbounded, 0), folded at compile
    // time); 2: the window (p.wl, p.wr).
    constexpr bool CAUSAL = MASK != 0;
    constexpr bool WIN = MASK == 2;  // left bound in use (every wl_ test is guarded by it)
    const int wl_ = MASK == 2 ? p.wl : kUnbounded;
    const int wr_ = MASK == 2 ? p.wr : 0;
    constexpr int G4 = D / 16;  // float4 groups per lane
    __shared__ __attribute__((aligned(16))) float Ks[kBN32 * D];
    __shared__ __attribute__((aligned(16))) float Vs[kBN32 * D];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int row = lane >> 2, part = lane & 3;
    const int units = p.B * p.Hq;
    const int slot = blockIdx.x / units;
    const int unit = blockIdx.x - slot * units;
    const int qb = CAUSAL ? p.nqb - 1 - slot : slot;
    const int b = unit / p.Hq, h = unit - (unit / p.Hq) * p.Hq;
    const int g = h / (p.Hq / p.Hkv);
    const SeqSpan sq = seq_span(p.cu, p.total, p.Hq, p.Hkv, p.N, b);
    const int N = sq.n;
    if (qb * kBM32 >= N) return;  // past the end of a shorter packed sequence (whole workgroup)
    const size_t qoff = sq.qrow(h) * D;
    const size_t kvoff = sq.kvrow(g) * D;
    const float* __restrict__ Qh = static_cast<const float*>(p.Q) + qoff;
    const float* __restrict__ Kh = static_cast<const float*>(p.K) + kvoff;
    const float* __restrict__ Vh = static_cast<const float*>(p.V) + kvoff;
    float* __restrict__ Oh = static_cast<float*>(p.O) + qoff;

    const int q0 = qb * kBM32;
    const int qrow = q0 + 16 * w + row;

    f32x4 q[G4], o[G4];
#pragma unroll
    for (int i = 0; i < G4; ++i) {
        q[i] = (qrow < N) ? *reinterpret_cast<const f32x4*>(Qh + size_t(qrow) * D + 16 * i + 4 * part) : f32x4{};
        o[i] = f32x4{};
    }
    float m = -INFINITY, l = 0.f;

    // masked kernels see keys q - wl .. q + wr of each query q
    const int kend = CAUSAL ? min(N, q0 + kBM32 + wr_) : N;
    const int kt0 = WIN ? max(0, q0 - wl_) / kBN32 : 0;
    const int ntiles = (kend + kBN32 - 1) / kBN32;
    for (int kt = kt0; kt < ntiles; ++kt) {
        const int kstart = kt * kBN32;
        __syncthreads();
        for (int idx = tid; idx < kBN32 * D / 4; idx += 256) {
            const int r = idx / (D / 4), c4 = idx % (D / 4);
            const int key = kstart + r;
            f32x4 kv = f32x4{}, vv = f32x4{};
            if (key < N) {
                kv = *reinterpret_cast<const f32x4*>(Kh + size_t(key) * D + 4 * c4);
                vv = *reinterpret_cast<const f32x4*>(Vh + size_t(key) * D + 4 * c4);
            }
            *reinterpret_cast<f32x4*>(Ks + r * D + 4 * c4) = kv;
            *reinterpret_cast<f32x4*>(Vs + r * D + 4 * c4) = vv;
        }
        __syncthreads();

        float s[kBN32];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBN32; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < G4; ++i) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(Ks + j * D + 16 * i + 4 * part);
                acc = fmaf(q[i][0], kv[0], acc);
                acc = fmaf(q[i][1], kv[1], acc);
                acc = fmaf(q[i][2], kv[2], acc);
                acc = fmaf(q[i][3], kv[3], acc);
            }
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            float t = acc * p.scale_log2;
            const int key = kstart + j;
            if ((CAUSAL && (key > qrow + wr_ || (WIN && key < qrow - wl_))) || key >= N) t = -INFINITY;
            s[j] = t;
            mx = fmaxf(mx, t);
        }
        const float m_new = fmaxf(m, mx);
        const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < G4; ++i) o[i] *= alpha;
#pragma unroll
        for (int j = 0; j < kBN32; ++j) {
            const float e = (s[j] == -INFINITY) ? 0.f : exp2f(s[j] - m_new);
            l += e;
#pragma unroll
            for (int i = 0; i < G4; ++i) {
                const f32x4 vv = *reinterpret_cast<const f32x4*>(Vs + j * D + 16 * i + 4 * part);
                o[i][0] = fmaf(e, vv[0], o[i][0]);
                o[i][1] = fmaf(e, vv[1], o[i][1]);
                o[i][2] = fmaf(e, vv[2], o[i][2]);
                o[i][3] = fmaf(e, vv[3], o[i][3]);
            }
        }
    }
    if (qrow < N) {
        const float inv = 1.f / l;
#pragma unroll
        for (int i = 0; i < G4; ++i)
            *reinterpret_cast<f32x4*>(Oh + size_t(qrow) * D + 16 * i + 4 * part) = o[i] * inv;
        if (part == 0 && p.LSE != nullptr) p.LSE[sq.qrow(h) + qrow] = (m + log2f(l)) * kLn2;
    }
}

template <int D, int MASK>
hipError_t launch_fwd_f32_t(FwdParams p, hipStream_t stream) {
    p.nqb = (p.N + kBM32 - 1) / kBM32;
    const long long blocks = (long long)p.nqb * p.B * p.Hq;
    hipLaunchKernelGGL((fwd_f32_kernel<D, MASK>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(FwdParams p, int d, int causal, hipStream_t stream) {
    const int mk = !causal ? 0 : (p.wl >= kUnbounded && p.wr == 0) ? 1 : 2;
#define FA_F32_DISPATCH(DD) \
    (mk == 0 ? launch_fwd_f32_t<DD, 0>(p, stream) : mk == 1 ? launch_fwd_f32_t<DD, 1>(p, stream) \
                                                            : launch_fwd_f32_t<DD, 2>(p, stream))
    switch (d) {
        case 64: return FA_F32_DISPATCH(64);
        case 128: return FA_F32_DISPATCH(128);
        case 256: return FA_F32_DISPATCH(256);
        default: return hipErrorInvalidValue;
    }
#undef FA_F32_DISPATCH
}

}  // namespace fa
