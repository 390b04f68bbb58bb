// Softmax of independent rows, y = softmax(scale * x) along each row of
// x [rows, n], with the row's log-sum-exp.
//
// The page "[Performance] [WebGPU] Proposal: Add an option to use online
// softmax instead of naive softmax" (§三-§五) contrasts the three-pass
// softmax (a pass for the maximum, one for the sum, one to normalise) with
// the online one, where a running maximum and a running sum rescaled by
// exp(m_old - m_new) come out of a single pass (chapter "2. 自注意力机制算子…",
// §2.3 and §2.6). Both are here:
//   * online: the threads of a row (64 to 1024, as few as hold it; rows of
//     at most 1024 values go 2 or 4 to a wave, with all their loads issued
//     together) keep the row in registers, 32 values each, up to 32768 per
//     row, so each element is read once and written once; with
//     the values on chip, the row max and then the row sum are plain
//     reductions. Longer rows stream twice: a pass of per-thread online
//     (m, l) updates over 16-byte chunks, the threads' pairs merged with
//     m = max, l = sum l_i 2^(m_i - m) (the online rule applied to blocks),
//     then a pass that writes y.
//   * three-pass: the maximum, the sum and the normalisation each read the
//     row again.
// Arithmetic in fp32, base-2 exponentials with scale*log2(e) folded in;
// entries equal to -inf get probability 0; a row with no finite entry gives
// y = 0 and lse = -inf. The output is rounded once to the storage type.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInfS = -__builtin_inff();
constexpr int SVALS = 32;  // row values per thread held in registers

struct SoftmaxParams {
    const void* x;
    void* y;
    float* lse;
    int64_t rows;
    int n;
    float c;  // scale * log2(e), > 0
};

// 16-byte chunk <-> fp32 values. NT: a non-temporal access, for data touched
// for the last time (the online kernels read x once and write y once; the
// three-pass kernel re-reads x and keeps it cached).
template <typename Tag> struct Chunk;
template <> struct Chunk<BF16> {
    static constexpr int E = 8;
    template <bool NT = false> __device__ static void load(const void* p, float (&v)[E]) {
        const u32x4* a = reinterpret_cast<const u32x4*>(p);
        const u32x4 w = NT ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = lo16<BF16>(w[i]); v[2 * i + 1] = hi16<BF16>(w[i]); }
    }
    template <bool NT = false> __device__ static void store(void* p, const float (&v)[E]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack2<BF16>(v[2 * i], v[2 * i + 1]);
        u32x4* a = reinterpret_cast<u32x4*>(p);
        if (NT) __builtin_nontemporal_store(w, a); else *a = w;
    }
};
template <> struct Chunk<F16> {
    static constexpr int E = 8;
    template <bool NT = false> __device__ static void load(const void* p, float (&v)[E]) {
        const u32x4* a = reinterpret_cast<const u32x4*>(p);
        const u32x4 w = NT ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[2 * i] = lo16<F16>(w[i]); v[2 * i + 1] = hi16<F16>(w[i]); }
    }
    template <bool NT = false> __device__ static void store(void* p, const float (&v)[E]) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack2<F16>(v[2 * i], v[2 * i + 1]);
        u32x4* a = reinterpret_cast<u32x4*>(p);
        if (NT) __builtin_nontemporal_store(w, a); else *a = w;
    }
};
template <> struct Chunk<F32> {
    static constexpr int E = 4;
    template <bool NT = false> __device__ static void load(const void* p, float (&v)[E]) {
        const f32x4* a = reinterpret_cast<const f32x4*>(p);
        const f32x4 w = NT ? __builtin_nontemporal_load(a) : *a;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = w[i];
    }
    template <bool NT = false> __device__ static void store(void* p, const float (&v)[E]) {
        const f32x4 w = {v[0], v[1], v[2], v[3]};
        f32x4* a = reinterpret_cast<f32x4*>(p);
        if (NT) __builtin_nontemporal_store(w, a); else *a = w;
    }
};

// (m, l) merge: the pair describing the union of two sets of values.
__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
    const float mm = fmaxf(m, m2);
    if (mm == kNegInfS) return;  // both empty
    l = (m == kNegInfS ? 0.f : l * fast_exp2(m - mm)) + (m2 == kNegInfS ? 0.f : l2 * fast_exp2(m2 - mm));
    m = mm;
}

// Reductions over the TPR threads of one row (TPR / 64 whole waves). `red`
// holds 2 floats per wave of the workgroup; every thread of the row gets the
// result.
template <int TPR> struct RowReduce {
    static constexpr int W = TPR / 64;  // waves per row
    __device__ static void merge(float& m, float& l, float* red) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float m2 = __shfl_xor(m, off, 64), l2 = __shfl_xor(l, off, 64);
            merge_ml(m, l, m2, l2);
        }
        if constexpr (W > 1) {
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
            const int w0 = wave - wave % W;  // first wave of this row
            if (lane == 0) { red[2 * wave] = m; red[2 * wave + 1] = l; }
            __syncthreads();
            m = red[2 * w0];
            l = red[2 * w0 + 1];
            for (int w = 1; w < W; ++w) merge_ml(m, l, red[2 * (w0 + w)], red[2 * (w0 + w) + 1]);
            __syncthreads();  // red is reused by a later call
        }
    }
    __device__ static float max(float m, float* red) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if constexpr (W > 1) {
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
            const int w0 = wave - wave % W;
            if (lane == 0) red[wave] = m;
            __syncthreads();
            m = red[w0];
            for (int w = 1; w < W; ++w) m = fmaxf(m, red[w0 + w]);
            __syncthreads();
        }
        return m;
    }
    __device__ static float sum(float l, float* red) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off, 64);
        if constexpr (W > 1) {
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
            const int w0 = wave - wave % W;
            if (lane == 0) red[wave] = l;
            __syncthreads();
            l = 0.f;
            for (int w = 0; w < W; ++w) l += red[w0 + w];
            __syncthreads();
        }
        return l;
    }
};

// A workgroup of NT threads serves NT / TPR rows, TPR threads each.
template <int TPR> constexpr int threads_of() { return TPR < 256 ? 256 : TPR; }

template <typename Tag, int TPR>
__global__ __launch_bounds__(threads_of<TPR>()) void softmax_online_kernel(SoftmaxParams p) {
    using C = Chunk<Tag>;
    using R = RowReduce<TPR>;
    constexpr int E = C::E;
    constexpr int EB = 16;          // bytes per chunk
    constexpr int SCH = SVALS / E;  // chunks per thread held in registers
    constexpr int NT = threads_of<TPR>();
    __shared__ float red[2 * NT / 64];
    const int64_t row = (int64_t)blockIdx.x * (NT / TPR) + threadIdx.x / TPR;
    const bool live = row < p.rows;  // the last workgroup may have spare rows
    // (every thread, live or not, takes the same path: the row reductions
    // contain workgroup barriers)
    const int nchunk = live ? p.n / E : 0;
    const unsigned char* xr = static_cast<const unsigned char*>(p.x) + row * (int64_t)p.n * (EB / E);
    unsigned char* yr = static_cast<unsigned char*>(p.y) + row * (int64_t)p.n * (EB / E);
    const int tid = threadIdx.x % TPR;
    float m = kNegInfS, l = 0.f;
    if (p.n / E <= TPR * SCH) {
        // the row stays in registers: one read, one write per element
        float v[SCH][E];
#pragma unroll
        for (int i = 0; i < SCH; ++i) {
            const int ci = tid + i * TPR;
            if (ci < nchunk) {
                C::template load<true>(xr + (int64_t)ci * EB, v[i]);
#pragma unroll
                for (int e = 0; e < E; ++e) { v[i][e] *= p.c; m = fmaxf(m, v[i][e]); }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[i][e] = kNegInfS;
            }
        }
        // with the row on chip, its max and then its sum are plain reductions
        m = R::max(m, red);
        if (m != kNegInfS) {
#pragma unroll
            for (int i = 0; i < SCH; ++i)
                if (tid + i * TPR < nchunk) {  // slots past the row hold nothing
#pragma unroll
                    for (int e = 0; e < E; ++e) l += fast_exp2(v[i][e] - m);
                }
        }
        l = R::sum(l, red);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float mu = m == kNegInfS ? 0.f : m;
#pragma unroll
        for (int i = 0; i < SCH; ++i) {
            const int ci = tid + i * TPR;
            if (ci < nchunk) {
                float o[E];
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = fast_exp2(v[i][e] - mu) * inv;
                C::template store<true>(yr + (int64_t)ci * EB, o);
            }
        }
    } else {
        // longer rows: per-thread online (m, l) over its chunks, then a
        // second read that writes the outputs
        for (int ci = tid; ci < nchunk; ci += TPR) {
            float v[E];
            C::load(xr + (int64_t)ci * EB, v);
            float mc = kNegInfS;
#pragma unroll
            for (int e = 0; e < E; ++e) { v[e] *= p.c; mc = fmaxf(mc, v[e]); }
            if (mc == kNegInfS) continue;
            float lc = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) lc += fast_exp2(v[e] - mc);
            merge_ml(m, l, mc, lc);
        }
        R::merge(m, l, red);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float mu = m == kNegInfS ? 0.f : m;
        for (int ci = tid; ci < nchunk; ci += TPR) {
            float v[E];
            C::template load<true>(xr + (int64_t)ci * EB, v);  // the last read
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = fast_exp2(v[e] * p.c - mu) * inv;
            C::template store<true>(yr + (int64_t)ci * EB, v);
        }
    }
    if (live && tid == 0 && p.lse != nullptr) p.lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInfS;
}

// Short rows (at most 64 * SVALS / RPW values): each wave holds RPW rows,
// one after another, issuing all their loads before any reduction, so that
// a wave keeps RPW times more bytes in flight; each row reduces across the
// wave's 64 lanes only (no barriers).
template <typename Tag, int RPW>
__global__ __launch_bounds__(256) void softmax_online_short_kernel(SoftmaxParams p) {
    using C = Chunk<Tag>;
    constexpr int E = C::E;
    constexpr int EB = 16;
    constexpr int SPR = SVALS / E / RPW;  // chunk slots per lane and row
    static_assert(SPR >= 1, "rows per wave exceed the register slots");
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    const int nch = p.n / E;
    float v[RPW][SPR][E];
    float m[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const bool live = row0 + r < p.rows;
        const unsigned char* xr = static_cast<const unsigned char*>(p.x) + (row0 + r) * (int64_t)p.n * (EB / E);
        m[r] = kNegInfS;
#pragma unroll
        for (int j = 0; j < SPR; ++j) {
            const int ci = lane + j * 64;
            if (live && ci < nch) {
                C::template load<true>(xr + (int64_t)ci * EB, v[r][j]);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) v[r][j][e] = kNegInfS;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
#pragma unroll
        for (int j = 0; j < SPR; ++j)
#pragma unroll
            for (int e = 0; e < E; ++e) { v[r][j][e] *= p.c; m[r] = fmaxf(m[r], v[r][j][e]); }
        m[r] = RowReduce<64>::max(m[r], nullptr);
    }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
        const bool live = row0 + r < p.rows;
        float l = 0.f;
        if (m[r] != kNegInfS) {
#pragma unroll
            for (int j = 0; j < SPR; ++j)
                if (lane + j * 64 < nch) {  // slots past the row hold nothing
#pragma unroll
                    for (int e = 0; e < E; ++e) l += fast_exp2(v[r][j][e] - m[r]);
                }
        }
        l = RowReduce<64>::sum(l, nullptr);
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const float mu = m[r] == kNegInfS ? 0.f : m[r];
        unsigned char* yr = static_cast<unsigned char*>(p.y) + (row0 + r) * (int64_t)p.n * (EB / E);
#pragma unroll
        for (int j = 0; j < SPR; ++j) {
            const int ci = lane + j * 64;
            if (live && ci < nch) {
                float o[E];
#pragma unroll
                for (int e = 0; e < E; ++e) o[e] = fast_exp2(v[r][j][e] - mu) * inv;
                C::template store<true>(yr + (int64_t)ci * EB, o);
            }
        }
        if (live && lane == 0 && p.lse != nullptr) p.lse[row0 + r] = l > 0.f ? (m[r] + log2f(l)) * kLn2 : kNegInfS;
    }
}

template <typename Tag, int TPR>
__global__ __launch_bounds__(threads_of<TPR>()) void softmax_three_pass_kernel(SoftmaxParams p) {
    using C = Chunk<Tag>;
    using R = RowReduce<TPR>;
    constexpr int E = C::E;
    constexpr int EB = 16;
    constexpr int NT = threads_of<TPR>();
    __shared__ float red[NT / 64];
    const int64_t row = (int64_t)blockIdx.x * (NT / TPR) + threadIdx.x / TPR;
    const bool live = row < p.rows;
    const int nchunk = live ? p.n / E : 0;
    const unsigned char* xr = static_cast<const unsigned char*>(p.x) + row * (int64_t)p.n * (EB / E);
    unsigned char* yr = static_cast<unsigned char*>(p.y) + row * (int64_t)p.n * (EB / E);
    const int tid = threadIdx.x % TPR;
    // pass 1: the maximum
    float m = kNegInfS;
    for (int ci = tid; ci < nchunk; ci += TPR) {
        float v[E];
        C::load(xr + (int64_t)ci * EB, v);
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, v[e] * p.c);
    }
    m = R::max(m, red);
    const float mu = m == kNegInfS ? 0.f : m;
    // pass 2: the sum
    float l = 0.f;
    for (int ci = tid; ci < nchunk; ci += TPR) {
        float v[E];
        C::load(xr + (int64_t)ci * EB, v);
#pragma unroll
        for (int e = 0; e < E; ++e) l += fast_exp2(v[e] * p.c - mu);
    }
    l = R::sum(l, red);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // pass 3: normalise
    for (int ci = tid; ci < nchunk; ci += TPR) {
        float v[E];
        C::load(xr + (int64_t)ci * EB, v);
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = fast_exp2(v[e] * p.c - mu) * inv;
        C::store(yr + (int64_t)ci * EB, v);
    }
    if (live && tid == 0 && p.lse != nullptr) p.lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : kNegInfS;
}

template <typename Tag, int TPR>
hipError_t launch_softmax_tpr(const SoftmaxParams& p, int mode, hipStream_t stream) {
    constexpr int NT = threads_of<TPR>();
    const int64_t grid = (p.rows + NT / TPR - 1) / (NT / TPR);
    if (mode == 0)
        hipLaunchKernelGGL((softmax_online_kernel<Tag, TPR>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
    else
        hipLaunchKernelGGL((softmax_three_pass_kernel<Tag, TPR>), dim3((unsigned)grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

// Threads per row: the fewest (64 .. 1024) that hold the row in registers,
// else 1024 streaming.
template <typename Tag>
hipError_t launch_softmax(const SoftmaxArgs& a, hipStream_t stream) {
    SoftmaxParams p;
    p.x = a.x;
    p.y = a.y;
    p.lse = a.lse;
    p.rows = a.rows;
    p.n = a.n;
    // c > 0 keeps -inf entries at probability 0; scale 0 runs as the limit
    // scale -> 0+ (uniform over the finite entries)
    p.c = a.scale > 0.f ? a.scale * kLog2e : 1e-30f;
    const int per_thread = SVALS;  // values per thread in registers
    const int64_t need = (a.n + per_thread - 1) / per_thread;
    if (a.mode == 0 && need <= 32) {
        // short rows: several per wave (4 waves, 4 * RPW rows per workgroup)
        const int rpw = need <= 16 ? 4 : 2;
        const int64_t grid = (p.rows + 4 * rpw - 1) / (4 * rpw);
        if (rpw == 4)
            hipLaunchKernelGGL((softmax_online_short_kernel<Tag, 4>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL((softmax_online_short_kernel<Tag, 2>), dim3((unsigned)grid), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    if (need <= 64) return launch_softmax_tpr<Tag, 64>(p, a.mode, stream);
    if (need <= 128) return launch_softmax_tpr<Tag, 128>(p, a.mode, stream);
    if (need <= 256) return launch_softmax_tpr<Tag, 256>(p, a.mode, stream);
    if (need <= 512) return launch_softmax_tpr<Tag, 512>(p, a.mode, stream);
    return launch_softmax_tpr<Tag, 1024>(p, a.mode, stream);
}

}  // namespace

hipError_t run_softmax_rows(const SoftmaxArgs& a, hipStream_t stream) {
    switch (a.dtype) {
    case 2: return launch_softmax<BF16>(a, stream);
    case 1: return launch_softmax<F16>(a, stream);
    default: return launch_softmax<F32>(a, stream);
    }
}

}  // namespace attn
