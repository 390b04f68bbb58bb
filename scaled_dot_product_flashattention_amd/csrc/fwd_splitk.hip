// Split-over-keys attention forward for few query rows over many keys (the
// single-query decode shape), where one workgroup per (batch, head) could not
// keep HBM busy.
//
// Kernel 1 cuts the keys of each query row into n_split equal ranges and
// gives each range to one workgroup. The workgroup streams its K/V rows once
// from HBM and keeps, per group of lanes, a running maximum m, a running sum
// l and an unnormalised weighted sum of V, rescaled by exp(m_old - m_new)
// whenever m grows (chapter "2. 自注意力机制算子…", §2.6). It then merges its
// lane groups and writes one partial (m, l, o[d]) to the workspace.
//
// Kernel 2 merges the n_split partials of each row with the block rule of the
// section "FlashAttention 分块计算原理与浏览器适配" of the WebGPU page:
// m = max_s m_s, weights exp(m_s - m), O = sum w_s o_s / sum w_s l_s.
//
// Layout of a partial in the workspace (fp32): [m, l, -, -, o_0 .. o_{d-1}],
// stride d + 4, indexed by (row = (b*H + h)*Sq + i) * n_split + split.
// m is kept in base-2 units of the scaled score (score * scale * log2 e).
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();

struct SplitParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* kv_len;
    float* ws;
    Strides sq;
    Strides sk;
    int B, H, Sq, Sk;
    float c;  // scale * log2(e)
    int causal;
    int n_split;
    int chunk;  // keys per split
};

__host__ __device__ constexpr int ws_stride(int d) { return d + 4; }

template <typename Tag, int D>
struct SplitCfg {
    static constexpr int ES = Tag::bytes;
    static constexpr int EPL = 16 / ES;     // elements of a row per lane (one 16-byte load)
    static constexpr int LPK = D / EPL;     // lanes per key row
    static constexpr int KPW = 64 / LPK;    // key rows per wave and load
    static constexpr int NW = 4;            // waves per workgroup
    static constexpr int U = 8;             // loads in flight per lane and tensor (8 measured 1.4 % faster than 4 and 6 on gfx950)
    static constexpr int KPI = NW * KPW * U;
    static constexpr int GROUPS = NW * KPW; // independent (m, l, o) states per workgroup
};

template <typename Tag>
__device__ __forceinline__ void unpack16(const u32x4& w, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = lo16<Tag>(w[e]);
        f[2 * e + 1] = hi16<Tag>(w[e]);
    }
}

template <typename Tag, int D>
__global__ __launch_bounds__(256) void splitk_partial_kernel(SplitParams p) {
    using C = SplitCfg<Tag, D>;
    using T = typename Tag::storage;
    constexpr int EPL = C::EPL;

    __shared__ float sm_m[C::GROUPS];
    __shared__ float sm_l[C::GROUPS];
    __shared__ float sm_o[C::GROUPS][D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane % C::LPK;  // which 16-byte slice of the row
    const int grp = lane / C::LPK;  // which key row of the wave's load

    int w = blockIdx.x;
    const int split = w % p.n_split;
    w /= p.n_split;
    const int h = w % p.H;
    const int bi = w / p.H;
    const int b = bi / p.Sq;
    const int i = bi - b * p.Sq;

    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const int lim = p.causal ? min(nb, i + 1) : nb;
    const int ks = split * p.chunk;
    const int ke = min(ks + p.chunk, lim);

    const T* qrow = static_cast<const T*>(p.q) + p.sq.head(b, h) + (int64_t)i * p.sq.s;
    const T* kb = static_cast<const T*>(p.k) + p.sk.head(b, h) + sub * EPL;
    const T* vb = static_cast<const T*>(p.v) + p.sk.head(b, h) + sub * EPL;

    float qf[EPL];
    {
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(qrow + sub * EPL);
        if constexpr (EPL == 8) {
            unpack16<Tag>(w4, qf);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) qf[e] = __uint_as_float(w4[e]);
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[e] *= p.c;
    }

    float m_run = kNegInf, l_run = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;

    for (int j0 = ks; j0 < ke; j0 += C::KPI) {
        u32x4 kr[C::U], vr[C::U];
        int jj[C::U];
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
            jj[u] = j0 + (u * C::NW + wave) * C::KPW + grp;
            const u32x4 z = {0u, 0u, 0u, 0u};
            // K and V are read exactly once: non-temporal loads keep them
            // out of the caches (measured 6.0 -> 6.8 TB/s at B8 H32 Sk32768)
            kr[u] = jj[u] < ke ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)jj[u] * p.sk.s)) : z;
            vr[u] = jj[u] < ke ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (int64_t)jj[u] * p.sk.s)) : z;
        }
        float x[C::U];
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
            float kf[EPL];
            if constexpr (EPL == 8) {
                unpack16<Tag>(kr[u], kf);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[e] = __uint_as_float(kr[u][e]);
            }
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
            x[u] = dot;
        }
        // sum the slices of each key row across its LPK lanes
#pragma unroll
        for (int off = C::LPK / 2; off >= 1; off >>= 1)
#pragma unroll
            for (int u = 0; u < C::U; ++u) x[u] += __shfl_xor(x[u], off);

        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
            x[u] = jj[u] < ke ? x[u] : kNegInf;
            mx = fmaxf(mx, x[u]);
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float pu[C::U];
        float rs = 0.f;
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
            pu[u] = fast_exp2(x[u] - m_use);
            rs += pu[u];
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
        for (int u = 0; u < C::U; ++u) {
            float vf[EPL];
            if constexpr (EPL == 8) {
                unpack16<Tag>(vr[u], vf);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) vf[e] = __uint_as_float(vr[u][e]);
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pu[u], vf[e], acc[e]);
        }
    }

    // ---- merge the GROUPS lane groups of this workgroup ----------------------
    const int gid = wave * C::KPW + grp;
    if (sub == 0) {
        sm_m[gid] = m_run;
        sm_l[gid] = l_run;
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm_o[gid][sub * EPL + e] = acc[e];
    __syncthreads();

    float* part = p.ws + ((int64_t)((b * p.H + h) * p.Sq + i) * p.n_split + split) * ws_stride(D);
    if (tid < D) {
        float M = kNegInf;
        for (int gg = 0; gg < C::GROUPS; ++gg) M = fmaxf(M, sm_m[gg]);
        const float M_use = (M == kNegInf) ? 0.f : M;
        float L = 0.f, A = 0.f;
        for (int gg = 0; gg < C::GROUPS; ++gg) {
            const float wgt = fast_exp2(sm_m[gg] - M_use);
            L = fmaf(wgt, sm_l[gg], L);
            A = fmaf(wgt, sm_o[gg][tid], A);
        }
        part[4 + tid] = A;
        if (tid == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

// Kernel 2. WPR waves per row (1 for many rows over few splits, 4 for few
// rows over many splits), 4 waves per workgroup. Every wave of a row first
// takes the row's max M over all splits' m (lane s reads m_s); wave j of the
// row then sums the splits s = j, j + WPR, ... with weights 2^(m_s - M), its
// lane holding elements EPL*lane .. EPL*lane + EPL-1 of o. With WPR > 1 the
// waves' sums meet in LDS. A split with nothing accumulated has m = -inf and
// weight 0; a row with no valid key gets O = 0 and LSE = -inf.
template <typename Tag, int D, int WPR>
__global__ __launch_bounds__(256) void splitk_merge_kernel(SplitParams p) {
    using T = typename Tag::storage;
    constexpr int EPL = D / 64;
    constexpr int RPB = 4 / WPR;  // rows per workgroup
    static_assert(D % 64 == 0 && 4 % WPR == 0, "merge shape");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % WPR;
    const int64_t rows = (int64_t)p.B * p.H * p.Sq;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool live = row < rows;
    const float* part = p.ws + (live ? row : 0) * p.n_split * ws_stride(D);

    float M = kNegInf;
    for (int s = lane; s < p.n_split; s += 64) M = fmaxf(M, part[(int64_t)s * ws_stride(D)]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float M_use = (M == kNegInf) ? 0.f : M;
    float L = 0.f;
    float A[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) A[e] = 0.f;
#pragma unroll 4
    for (int s = sub; s < p.n_split; s += WPR) {
        const float* ps = part + (int64_t)s * ws_stride(D);
        const float wgt = fast_exp2(ps[0] - M_use);
        L = fmaf(wgt, ps[1], L);
#pragma unroll
        for (int e = 0; e < EPL; ++e) A[e] = fmaf(wgt, ps[4 + EPL * lane + e], A[e]);
    }
    if constexpr (WPR > 1) {
        __shared__ float red[4][EPL * 64 + 1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) red[wave][EPL * lane + e] = A[e];
        if (lane == 0) red[wave][EPL * 64] = L;
        __syncthreads();
        if (sub == 0) {
            for (int j = 1; j < WPR; ++j) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) A[e] += red[wave + j][EPL * lane + e];
                L += red[wave + j][EPL * 64];
            }
        }
    }
    if (!live || sub != 0) return;
    const int i = (int)(row % p.Sq);
    const int h = (int)((row / p.Sq) % p.H);
    const int b = (int)(row / ((int64_t)p.Sq * p.H));
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T* orow = static_cast<T*>(p.o) + p.sq.head(b, h) + (int64_t)i * p.sq.s;
#pragma unroll
    for (int e = 0; e < EPL; ++e) orow[EPL * lane + e] = to_storage<Tag>(A[e] * inv);
    if (lane == 0 && p.lse != nullptr) p.lse[row] = L > 0.f ? (M + log2f(L)) * kLn2 : kNegInf;
}

// The merge for (rows, n_split): four waves per row when few rows share many
// splits, one otherwise.
template <typename Tag, int D>
hipError_t launch_merge_kernel(const SplitParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.B * p.H * p.Sq;
    if (rows > 0x7fffffff) return hipErrorInvalidValue;
    if (p.n_split >= 16 && rows < 4096)
        hipLaunchKernelGGL((splitk_merge_kernel<Tag, D, 4>), dim3((unsigned)rows), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((splitk_merge_kernel<Tag, D, 1>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                           stream, p);
    return hipGetLastError();
}

template <typename Tag, int D>
hipError_t launch_splitk(const FwdArgs& a, int n_split, void* workspace, hipStream_t stream) {
    SplitParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.kv_len = a.kv_len;
    p.ws = static_cast<float*>(workspace);
    p.sq = make_strides(a.layout, a.H, a.Sq, a.d);
    p.sk = make_strides(a.layout, a.H, a.Sk, a.d);
    p.B = a.B;
    p.H = a.H;
    p.Sq = a.Sq;
    p.Sk = a.Sk;
    p.c = a.scale * kLog2e;
    p.causal = a.causal ? 1 : 0;
    p.n_split = n_split;
    p.chunk = (a.Sk + n_split - 1) / n_split;
    const int64_t rows = (int64_t)a.B * a.H * a.Sq;
    const int64_t grid = rows * n_split;
    if (grid > 0x7fffffff || rows > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((splitk_partial_kernel<Tag, D>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_merge_kernel<Tag, D>(p, stream);
}

template <typename Tag, int D>
hipError_t launch_merge(const FwdArgs& a, int n_split, const void* workspace, hipStream_t stream) {
    SplitParams p = {};
    p.o = a.o;
    p.lse = a.lse;
    p.ws = static_cast<float*>(const_cast<void*>(workspace));
    p.sq = make_strides(a.layout, a.H, a.Sq, a.d);
    p.B = a.B;
    p.H = a.H;
    p.Sq = a.Sq;
    p.n_split = n_split;
    return launch_merge_kernel<Tag, D>(p, stream);
}

}  // namespace

hipError_t run_splitk_merge(const FwdArgs& a, int n_split, const void* workspace, hipStream_t stream) {
    switch (a.dtype) {
    case 2: return a.d == 64 ? launch_merge<BF16, 64>(a, n_split, workspace, stream)
                             : launch_merge<BF16, 128>(a, n_split, workspace, stream);
    case 1: return a.d == 64 ? launch_merge<F16, 64>(a, n_split, workspace, stream)
                             : launch_merge<F16, 128>(a, n_split, workspace, stream);
    default: return a.d == 64 ? launch_merge<F32, 64>(a, n_split, workspace, stream)
                              : launch_merge<F32, 128>(a, n_split, workspace, stream);
    }
}

size_t splitk_workspace_bytes(int B, int H, int Sq, int d, int n_split) {
    return (size_t)B * H * Sq * (size_t)n_split * ws_stride(d) * sizeof(float);
}

hipError_t run_splitk(const FwdArgs& a, int n_split, void* workspace, hipStream_t stream) {
    switch (a.dtype) {
    case 2:
        return a.d == 64 ? launch_splitk<BF16, 64>(a, n_split, workspace, stream)
                         : launch_splitk<BF16, 128>(a, n_split, workspace, stream);
    case 1:
        return a.d == 64 ? launch_splitk<F16, 64>(a, n_split, workspace, stream)
                         : launch_splitk<F16, 128>(a, n_split, workspace, stream);
    default:
        return a.d == 64 ? launch_splitk<F32, 64>(a, n_split, workspace, stream)
                         : launch_splitk<F32, 128>(a, n_split, workspace, stream);
    }
}

}  // namespace attn
