// Unfused attention baseline: the "standard implementation" of §2.5 of the
// chapter "2. 自注意力机制算子…以及FlashAttention优化", kept as a measuring stick
// for the fused kernel. Three launches, two materialised [Sq, Sk] matrices per
// (batch, head):
//   1. S = scale * Q K^T            (matrix cores; fp32 scores to scratch)
//   2. P = softmax(S) row by row    (the three-step softmax of §2.3: a pass
//      for the row max, a pass for the sum of shifted exponentials, a pass
//      that normalises; masked keys get P = 0) plus LSE
//   3. O = P V                      (matrix cores; P in the input type)
// S is kept in fp32: a 16-bit score loses up to a few percent of a
// probability at |s| ~ 16, which the parity bar does not allow.
// Scratch rows are padded to a multiple of 64 keys (ldS).
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();

struct NaiveParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* kv_len;
    float* S;
    void* P;
    Strides sq;
    Strides sk;
    int B, H, Sq, Sk;
    int64_t ldS;
    float scale;
    int causal;
    int n_qtiles;
    int n_ktiles;
};

constexpr int BM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int BN = 64;   // keys per tile

__host__ __device__ inline int64_t naive_ld(int Sk) { return ((int64_t)Sk + 63) / 64 * 64; }

// ---- 1. scores ------------------------------------------------------------
template <typename Tag, int D>
__global__ __launch_bounds__(256) void naive_scores_kernel(NaiveParams p) {
    using T = typename Tag::storage;
    constexpr int ES = Tag::bytes;
    constexpr bool k16 = ES == 2;
    constexpr int EPC = 16 / ES;
    constexpr int CPR = D / EPC;
    constexpr int KROW = D + EPC;
    __shared__ __align__(16) T Ks[BN * KROW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    int w = blockIdx.x;
    const int kt = w % p.n_ktiles;
    w /= p.n_ktiles;
    const int qt = w % p.n_qtiles;
    const int bh = w / p.n_qtiles;
    const int b = bh / p.H, h = bh % p.H;
    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const T* qp = static_cast<const T*>(p.q) + p.sq.head(b, h);
    const T* kp = static_cast<const T*>(p.k) + p.sk.head(b, h);

    for (int idx = tid; idx < BN * CPR; idx += 256) {
        const int row = idx / CPR, cc = idx % CPR;
        const int key = kt * BN + row;
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Ks + row * KROW + cc * EPC) =
            key < nb ? *reinterpret_cast<const u32x4*>(kp + (int64_t)key * p.sk.s + cc * EPC) : z;
    }
    __syncthreads();

    const int qi = qt * BM + wave * 32 + n32;
    const bool ok = qi < p.Sq;
    const T* qrow = qp + (int64_t)(ok ? qi : 0) * p.sq.s;
    f32x16 acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[kb][r] = 0.f;
    if constexpr (k16) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 bq = ok ? *reinterpret_cast<const u32x4*>(qrow + s * 16 + hh * 8) : z;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(Ks + (kb * 32 + n32) * KROW + s * 16 + hh * 8);
                acc[kb] = mfma16<Tag>(a, bq, acc[kb]);
            }
        }
    } else {
#pragma unroll 8
        for (int s = 0; s < D / 2; ++s) {
            const float bq = ok ? qrow[2 * s + hh] : 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) acc[kb] = mfma_f32(Ks[(kb * 32 + n32) * KROW + 2 * s + hh], bq, acc[kb]);
        }
    }
    if (!ok) return;
    float* srow = p.S + ((int64_t)bh * p.Sq + qi) * p.ldS + kt * BN;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const f32x4 v4 = {acc[kb][4 * jj] * p.scale, acc[kb][4 * jj + 1] * p.scale,
                              acc[kb][4 * jj + 2] * p.scale, acc[kb][4 * jj + 3] * p.scale};
            *reinterpret_cast<f32x4*>(srow + kb * 32 + 8 * jj + 4 * hh) = v4;
        }
}

// ---- 2. three-step softmax per row ------------------------------------------
__device__ __forceinline__ float block_reduce(float x, bool is_max, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float y = __shfl_xor(x, off);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = x;
    __syncthreads();
    x = red[0];
#pragma unroll
    for (int wv = 1; wv < 4; ++wv) x = is_max ? fmaxf(x, red[wv]) : x + red[wv];
    return x;
}

template <typename Tag>
__global__ __launch_bounds__(256) void naive_softmax_kernel(NaiveParams p) {
    using T = typename Tag::storage;
    __shared__ float red[4];
    const int row = blockIdx.x;  // (b*H + h)*Sq + i
    const int i = row % p.Sq;
    const int b = row / (p.Sq * p.H);
    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const int lim = p.causal ? min(nb, i + 1) : nb;
    const float* s = p.S + (int64_t)row * p.ldS;
    T* prow = static_cast<T*>(p.P) + (int64_t)row * p.ldS;

    float m = kNegInf;  // step 1: row maximum
    for (int j = threadIdx.x; j < lim; j += 256) m = fmaxf(m, s[j]);
    m = block_reduce(m, true, red);
    float l = 0.f;  // step 2: sum of shifted exponentials
    for (int j = threadIdx.x; j < lim; j += 256) l += fast_exp2((s[j] - m) * kLog2e);
    l = block_reduce(l, false, red);
    const float inv = lim > 0 ? 1.f / l : 0.f;  // step 3: normalise
    for (int j = threadIdx.x; j < p.ldS; j += 256)
        prow[j] = to_storage<Tag>(j < lim ? fast_exp2((s[j] - m) * kLog2e) * inv : 0.f);
    if (threadIdx.x == 0 && p.lse != nullptr) p.lse[row] = lim > 0 ? m + logf(l) : kNegInf;
}

// ---- 3. O = P V ---------------------------------------------------------------
template <typename Tag, int D>
__global__ __launch_bounds__(256) void naive_pv_kernel(NaiveParams p) {
    using T = typename Tag::storage;
    constexpr int ES = Tag::bytes;
    constexpr bool k16 = ES == 2;
    constexpr int EPC = 16 / ES;
    constexpr int CPR = D / EPC;
    constexpr int VROW = BN + 8 / ES;
    constexpr int OROW = D + EPC;
    constexpr int V_BYTES = D * VROW * ES;
    constexpr int O_BYTES = BM * OROW * ES;
    __shared__ __align__(16) unsigned char smem[V_BYTES > O_BYTES ? V_BYTES : O_BYTES];
    T* Vt = reinterpret_cast<T*>(smem);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n32 = lane & 31, hh = lane >> 5;
    const int qt = blockIdx.x % p.n_qtiles;
    const int bh = blockIdx.x / p.n_qtiles;
    const int b = bh / p.H, h = bh % p.H;
    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const int q_end = min((qt + 1) * BM, p.Sq);
    const int kend = p.causal ? min(nb, q_end) : nb;
    const T* vp = static_cast<const T*>(p.v) + p.sk.head(b, h);
    T* op = static_cast<T*>(p.o) + p.sq.head(b, h);
    const int qw0 = qt * BM + wave * 32;
    const int qi = qw0 + n32;
    const bool ok = qi < p.Sq;
    const T* prow = static_cast<const T*>(p.P) + ((int64_t)bh * p.Sq + (ok ? qi : 0)) * p.ldS;

    f32x16 acc[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    for (int t = 0; t * BN < kend; ++t) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        if constexpr (k16) {
            for (int idx = tid; idx < (BN / 2) * CPR; idx += 256) {
                const int pr = idx / CPR, cc = idx % CPR;
                const int key = t * BN + 2 * pr;
                const u32x4 r0 = key < nb ? *reinterpret_cast<const u32x4*>(vp + (int64_t)key * p.sk.s + cc * EPC) : z;
                const u32x4 r1 = key + 1 < nb ? *reinterpret_cast<const u32x4*>(vp + (int64_t)(key + 1) * p.sk.s + cc * EPC) : z;
                store_pair_transposed(Vt, VROW, cc, pr, r0, r1);
            }
        } else {
            for (int idx = tid; idx < BN * CPR; idx += 256) {
                const int row = idx / CPR, cc = idx % CPR;
                const int key = t * BN + row;
                const u32x4 r0 = key < nb ? *reinterpret_cast<const u32x4*>(vp + (int64_t)key * p.sk.s + cc * EPC) : z;
#pragma unroll
                for (int e = 0; e < 4; ++e) reinterpret_cast<uint32_t*>(Vt)[(cc * 4 + e) * VROW + row] = r0[e];
            }
        }
        __syncthreads();
        if (qw0 < p.Sq) {
            if constexpr (k16) {
                // contraction slot (lane half h, element e) <-> key 16u + 8h + e
#pragma unroll
                for (int u = 0; u < BN / 16; ++u) {
                    const u32x4 bp = ok ? *reinterpret_cast<const u32x4*>(prow + t * BN + 16 * u + 8 * hh) : z;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const T* vr = Vt + (db * 32 + n32) * VROW + 16 * u + 8 * hh;
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 4);
                        acc[db] = mfma16<Tag>(u32x4{lo[0], lo[1], hi[0], hi[1]}, bp, acc[db]);
                    }
                }
            } else {
#pragma unroll 8
                for (int u = 0; u < BN / 2; ++u) {
                    const float bp = ok ? prow[t * BN + 2 * u + hh] : 0.f;
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
                        acc[db] = mfma_f32(Vt[(db * 32 + n32) * VROW + 2 * u + hh], bp, acc[db]);
                }
            }
        }
        __syncthreads();
    }

    // O^T registers -> LDS [query][d] -> coalesced rows
    T* Os = reinterpret_cast<T*>(smem);
    T* orow = Os + (wave * 32 + n32) * OROW;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int d0 = db * 32 + 8 * jj + 4 * hh;
            if constexpr (k16) {
                *reinterpret_cast<u32x2*>(orow + d0) =
                    u32x2{pack2<Tag>(acc[db][4 * jj], acc[db][4 * jj + 1]),
                          pack2<Tag>(acc[db][4 * jj + 2], acc[db][4 * jj + 3])};
            } else {
                *reinterpret_cast<f32x4*>(orow + d0) =
                    f32x4{acc[db][4 * jj], acc[db][4 * jj + 1], acc[db][4 * jj + 2], acc[db][4 * jj + 3]};
            }
        }
    __syncthreads();
    for (int cidx = tid; cidx < BM * CPR; cidx += 256) {
        const int row = cidx / CPR, cc = cidx % CPR;
        const int q = qt * BM + row;
        if (q < p.Sq)
            *reinterpret_cast<u32x4*>(op + (int64_t)q * p.sq.s + cc * EPC) =
                *reinterpret_cast<const u32x4*>(Os + row * OROW + cc * EPC);
    }
}

template <typename Tag, int D>
hipError_t launch_naive(const FwdArgs& a, void* scratch, hipStream_t stream) {
    NaiveParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.kv_len = a.kv_len;
    p.ldS = naive_ld(a.Sk);
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    p.S = static_cast<float*>(scratch);
    p.P = static_cast<unsigned char*>(scratch) + rows * p.ldS * (int64_t)sizeof(float);
    p.sq = make_strides(a.layout, a.H, a.Sq, a.d);
    p.sk = make_strides(a.layout, a.H, a.Sk, a.d);
    p.B = a.B;
    p.H = a.H;
    p.Sq = a.Sq;
    p.Sk = a.Sk;
    p.scale = a.scale;
    p.causal = a.causal ? 1 : 0;
    p.n_qtiles = (a.Sq + BM - 1) / BM;
    p.n_ktiles = (int)(p.ldS / BN);
    const int64_t g1 = (int64_t)p.n_qtiles * p.n_ktiles * a.B * a.H;
    const int64_t g3 = (int64_t)p.n_qtiles * a.B * a.H;
    if (g1 > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((naive_scores_kernel<Tag, D>), dim3((unsigned)g1), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((naive_softmax_kernel<Tag>), dim3((unsigned)rows), dim3(256), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((naive_pv_kernel<Tag, D>), dim3((unsigned)g3), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

size_t naive_scratch_bytes(int B, int H, int Sq, int Sk, int dtype) {
    const int es = dtype == 0 ? 4 : 2;
    return (size_t)B * H * Sq * (size_t)naive_ld(Sk) * (sizeof(float) + es);
}

hipError_t run_naive(const FwdArgs& a, void* scratch, hipStream_t stream) {
    switch (a.dtype) {
    case 2:
        return a.d == 64 ? launch_naive<BF16, 64>(a, scratch, stream) : launch_naive<BF16, 128>(a, scratch, stream);
    case 1:
        return a.d == 64 ? launch_naive<F16, 64>(a, scratch, stream) : launch_naive<F16, 128>(a, scratch, stream);
    default:
        return a.d == 64 ? launch_naive<F32, 64>(a, scratch, stream) : launch_naive<F32, 128>(a, scratch, stream);
    }
}

}  // namespace attn
