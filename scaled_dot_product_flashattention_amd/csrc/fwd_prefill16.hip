// Fused attention forward for bf16 / fp16 inputs: one kernel, scores and
// probabilities stay on chip.
//
// Method (chapter "2. 自注意力机制算子…以及FlashAttention优化", §2.6, and the
// section "FlashAttention 分块计算原理与浏览器适配" of the WebGPU page): the
// queries of one head are cut into tiles of BM rows, the keys/values into
// tiles of BN rows. A workgroup owns one query tile, streams every key/value
// tile it needs through LDS, and keeps per query row a running maximum m and a
// running sum l; when m grows, the sum and the partial output are multiplied
// by exp(m_old - m_new) first. The output is divided by l once, at the end.
//
// Mapping to gfx950:
//   * 4 waves per workgroup, each owning 32*NQ query rows.
//   * Scores are computed transposed, S^T = K Q^T, on 32x32x16 matrix-core
//     blocks: a lane owns one query (its column) and half the keys of each
//     32-key block (its rows), so row max and row sum are in-lane but for one
//     exchange between the two lane halves (v_permlane32_swap).
//   * The output is kept transposed too, O^T += V^T P^T: probabilities feed
//     the second product straight from the score registers (rounded and
//     packed in pairs), and the rescale touches only the lane's own query.
//   * K and V tiles travel global -> LDS by direct DMA loads
//     (global_load_lds_dwordx4) into an NST-stage ring, NST-1 tiles ahead of
//     the one being computed; no registers are spent on staging. Both sit in
//     LDS row-major with their 16-byte chunks XOR-swizzled per row so that
//     the K operand reads (ds_read_b128) and the transposing V operand reads
//     (ds_read_b64_tr_b16) are free of bank conflicts.
//   * PIPE: the scores of tile t+1 are issued before the softmax of tile t.
//   * The running max moves lazily (only when a tile beats it by more than
//     2^8), so most tiles skip the rescale of the partial output; the result
//     is the same up to rounding because m, l and O always share one m.
//   * Workgroups of one head stay on one XCD (its L2 then serves every re-read
//     of that head's K/V); causal tiles start longest-first.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();
// The running max moves only when a tile's max exceeds it by more than this
// (base-2 units): probabilities then stay below 2^8.
constexpr float kLazyRescale = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct Prefill16Params {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* kv_len;
    Strides sq;  // q and o
    Strides sk;  // k and v
    int B, H, Sq, Sk;
    float c;  // scale * log2(e)
    int causal;
    int n_qtiles;
    int remap;  // grid size is a multiple of 8: keep each head's tiles on one XCD
};

// XOR swizzle of the 16-byte chunks of LDS row `row` (see the header comment).
template <int D> __device__ __forceinline__ int swz_k(int row) {
    return D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int D> __device__ __forceinline__ int swz_v(int row) {
    return D == 64 ? (((row >> 1) & 1) << 2) : ((row & 3) << 2);
}

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at LDS address lds_addr + 16*l; lds_addr is wave-uniform
// (it travels in M0). Issued from asm so that the compiler neither counts it
// nor adds its own waits before LDS reads: the kernel waits for these loads
// explicitly with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr) : "memory");
}

// Workgroup barrier without a memory fence: each wave has already waited for
// its own DMA loads; the empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename Tag, int D, int NQ, int BN, int NST, bool PIPE>
__global__ __launch_bounds__(256, 2) void fwd_prefill16_kernel(Prefill16Params p) {
    constexpr int NW = 4;
    constexpr int BM = NW * 32 * NQ;
    constexpr int RB = D * 2;                      // bytes per K/V row
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int TILE_B = BN * RB;
    constexpr int STAGE_B = 2 * TILE_B;            // K tile, then V tile
    constexpr int DMA1 = TILE_B / 16 / 256;        // DMA loads per thread, tensor and tile
    constexpr int DPT = 2 * DMA1;                  // ... for K and V
    constexpr int P = NST - 1;                     // tiles in flight ahead
    constexpr int OROW = D + 8;                    // output staging row (elements)
    constexpr int OUT_B = NW * 32 * NQ * OROW * 2;
    constexpr int LDS_B = NST * STAGE_B > OUT_B ? NST * STAGE_B : OUT_B;
    static_assert(DMA1 >= 1 && TILE_B % (16 * 256) == 0, "tile must split over 256 lanes");
    static_assert(P >= (PIPE ? 2 : 1), "pipelining needs a deeper ring");
    static_assert(P * DPT < 64, "vmcnt range");
    using T = uint16_t;

    __shared__ __align__(16) unsigned char smem[LDS_B];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n32 = lane & 31;
    const int hh = lane >> 5;

    // ---- which (batch, head, query tile) ---------------------------------
    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int w = p.remap ? (g & 7) * (G >> 3) + (g >> 3) : g;
    const int bh = w / p.n_qtiles;
    int qt = w - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest causal tiles first
    const int b = bh / p.H;
    const int h = bh - b * p.H;

    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const int q0 = qt * BM;
    const int q_end = min(q0 + BM, p.Sq);
    const int kend = p.causal ? min(nb, q_end) : nb;  // keys any row of the tile can see
    const int ntiles = (kend + BN - 1) / BN;

    const T* qp = static_cast<const T*>(p.q) + b * p.sq.b + h * p.sq.h;
    const T* kp = static_cast<const T*>(p.k) + b * p.sk.b + h * p.sk.h;
    const T* vp = static_cast<const T*>(p.v) + b * p.sk.b + h * p.sk.h;
    T* op = static_cast<T*>(p.o) + b * p.sq.b + h * p.sq.h;

    const int qw0 = q0 + wave * 32 * NQ;  // first query row of this wave
    const bool wave_active = qw0 < p.Sq;
    const int wave_kend = p.causal ? min(nb, min(qw0 + 32 * NQ, p.Sq)) : nb;
    const int wave_lim_min = p.causal ? min(nb, qw0 + 1) : nb;  // tiles past this need masks
    auto active = [&](int tile) { return wave_active && tile * BN < wave_kend; };

    // ---- Q operands (B of S^T = K Q^T), in registers for the whole loop ----
    // K-step s holds q[row][16s + 8h .. +7].
    u32x4 qop[NQ][D / 16];
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        const int qi = qw0 + gq * 32 + n32;
        const bool ok = qi < p.Sq;
        const T* row = qp + (int64_t)(ok ? qi : 0) * p.sq.s;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            qop[gq][s] = ok ? *reinterpret_cast<const u32x4*>(row + s * 16 + hh * 8) : z;
        }
    }
    wait_vmcnt<0>();  // Q is in registers before any DMA load is in flight

    // ---- DMA of one K/V tile into LDS stage tile % NST ----------------------
    // Thread-slot i*256 + tid of the tile is the 16-byte chunk (row, pc); it
    // holds the logical chunk pc ^ swz(row) of key row `row`. Rows at or past
    // the valid length reread the last valid row (finite, masked later). The
    // per-thread offsets do not depend on the tile and are computed once.
    int64_t koff[DMA1], voff[DMA1];
#pragma unroll
    for (int i = 0; i < DMA1; ++i) {
        const int slot = i * 256 + tid;
        const int row = slot / CPR, pc = slot - row * CPR;
        koff[i] = row * p.sk.s + (pc ^ swz_k<D>(row)) * 8;
        voff[i] = row * p.sk.s + (pc ^ swz_v<D>(row)) * 8;
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
    auto issue_tile = [&](int tile) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + (tile % NST) * STAGE_B + wave * 1024);
        const int key0 = tile * BN;
        if (key0 + BN <= nb) {
            const T* kt = kp + key0 * p.sk.s;
            const T* vt = vp + key0 * p.sk.s;
#pragma unroll
            for (int i = 0; i < DMA1; ++i) {
                dma16(kt + koff[i], st + i * 4096);
                dma16(vt + voff[i], st + i * 4096 + TILE_B);
            }
        } else {
#pragma unroll
            for (int i = 0; i < DMA1; ++i) {
                const int slot = i * 256 + tid;
                const int row = slot / CPR, pc = slot - row * CPR;
                const int64_t key = min(key0 + row, nb - 1);
                dma16(kp + key * p.sk.s + (pc ^ swz_k<D>(row)) * 8, st + i * 4096);
                dma16(vp + key * p.sk.s + (pc ^ swz_v<D>(row)) * 8, st + i * 4096 + TILE_B);
            }
        }
    };
    // wait until at most n_after tiles' DMA loads (issued after the awaited
    // tile) are still in flight
    auto wait_tiles = [&](int n_after) {
        if constexpr (P >= 3) {
            if (n_after >= 2) { wait_vmcnt<(P >= 3 ? 2 * DPT : 0)>(); return; }
        }
        if constexpr (P >= 2) {
            if (n_after >= 1) { wait_vmcnt<(P >= 2 ? DPT : 0)>(); return; }
        }
        wait_vmcnt<0>();
    };

    // ---- operand reads ----------------------------------------------------------
    auto stage = [&](int tile) { return smem + (tile % NST) * STAGE_B; };
    auto k_operand = [&](const unsigned char* kt, int kb, int s) -> u32x4 {
        const int row = kb * 32 + n32;
        const int lc = 2 * s + hh;
        return *reinterpret_cast<const u32x4*>(kt + row * RB + ((lc ^ swz_k<D>(row)) << 4));
    };
    // V^T operand of block (kb, u, db): lane (d = db*32 + l%32, half h) needs
    // V[kb*32 + 16u + 4h + e][d] and V[kb*32 + 16u + 8 + 4h + e][d], e = 0..3.
    // ds_read_b64_tr_b16 gives lane i of each 16-lane group element (i % 4) of
    // the 8-byte piece addressed by lane 4e + i/4 of the group, as element e.
    const int grp = lane >> 4;
    const int e_tr = (lane & 15) >> 2;
    const int q_tr = lane & 3;
    auto v_operand = [&](const unsigned char* vt, int kb, int u, int db) -> u32x4 {
        u32x2 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int row = kb * 32 + 16 * u + 8 * hf + 4 * hh + e_tr;
            const int lc = db * 4 + 2 * (grp & 1) + (q_tr >> 1);
            const unsigned char* a = vt + row * RB + ((lc ^ swz_v<D>(row)) << 4) + 8 * (q_tr & 1);
            const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
            part[hf] = __builtin_bit_cast(u32x2, r);
        }
        return u32x4{part[0][0], part[0][1], part[1][0], part[1][1]};
    };

    // ---- running state -----------------------------------------------------
    f32x16 oacc[NQ][D / 32];
    float m_run[NQ], l_run[NQ];
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        m_run[gq] = kNegInf;
        l_run[gq] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[gq][db][r] = 0.f;
    }
    const float c = p.c;

    auto qk_tile = [&](const unsigned char* kt, f32x16 (&sacc)[BN / 32][NQ]) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][gq][r] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                const u32x4 a = k_operand(kt, kb, s);
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) sacc[kb][gq] = mfma16<Tag>(a, qop[gq][s], sacc[kb][gq]);
            }
        }
    };

    // pq[gq][kb][u]: B operand of the (kb, u) product, the probabilities of
    // result registers 8u .. 8u+7 rounded and packed in pairs
    u32x4 pq[NQ][BN / 32][2];
    auto softmax_tile = [&](auto masked_tag, f32x16 (&sacc)[BN / 32][NQ], int tile, float (&alpha_out)[NQ], bool& rescale) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
            if constexpr (MASKED) {
                const int qi = qw0 + gq * 32 + n32;
                const int lim = p.causal ? min(nb, qi + 1) : nb;
#pragma unroll
                for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (tile * BN + kb * 32 + blk_row(r, hh) >= lim) sacc[kb][gq][r] = kNegInf;
            }
            float mq[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 8) {
                    const int ch = (kb * 2 + r / 8) & 3;
                    mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r], sacc[kb][gq][r + 1]));
                    mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r + 2], sacc[kb][gq][r + 3]));
                    mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r + 4], sacc[kb][gq][r + 5]));
                    mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r + 6], sacc[kb][gq][r + 7]));
                }
            float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
            mx = fmaxf(mx, swap_halves(mx));
            const float mxs = (MASKED && mx == kNegInf) ? kNegInf : mx * c;
            alpha_out[gq] = 1.f;
            if (__any(mxs > m_run[gq] + kLazyRescale)) {
                const float m_new = fmaxf(m_run[gq], mxs);
                const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[gq] - m_new);
                m_run[gq] = m_new;
                l_run[gq] *= alpha;
                alpha_out[gq] = alpha;
                rescale = true;
            }
            const float m_use = (m_run[gq] == kNegInf) ? 0.f : m_run[gq];
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float x0 = sacc[kb][gq][r], x1 = sacc[kb][gq][r + 1];
                    float p0 = fast_exp2(fmaf(x0, c, -m_use));
                    float p1 = fast_exp2(fmaf(x1, c, -m_use));
                    if constexpr (MASKED) {
                        p0 = (x0 == kNegInf) ? 0.f : p0;
                        p1 = (x1 == kNegInf) ? 0.f : p1;
                    }
                    const uint32_t w2 = pack2<Tag>(p0, p1);
                    pq[gq][kb][r / 8][(r / 2) & 3] = w2;
                    rs[(r / 2) & 3] = dot2_sum<Tag>(w2, rs[(r / 2) & 3]);
                }
            l_run[gq] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        }
    };

    auto pv_tile = [&](const unsigned char* vt) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x4 a = v_operand(vt, kb, u, db);
#pragma unroll
                    for (int gq = 0; gq < NQ; ++gq) oacc[gq][db] = mfma16<Tag>(a, pq[gq][kb][u], oacc[gq][db]);
                }
    };

    // ---- key loop over the DMA ring ---------------------------------------------
    // Unrolled by two so the score registers of tiles t and t+1 alternate
    // between two fixed sets instead of being copied.
    constexpr int AHEAD = PIPE ? 1 : 0;  // tiles needed beyond the one softmaxed
    auto step = [&](int t, f32x16 (&s_now)[BN / 32][NQ], f32x16 (&s_nxt)[BN / 32][NQ]) {
        const int last_issued = min(t + P - 1, ntiles - 1);
        const int need = min(t + AHEAD, ntiles - 1);
        wait_tiles(last_issued - need);
        barrier_nofence();  // tiles <= need are in LDS; every wave is done with tile t-1
        if (t + P < ntiles) issue_tile(t + P);  // into the stage of tile t-1
        if constexpr (PIPE) {
            if (t + 1 < ntiles && active(t + 1)) qk_tile(stage(t + 1), s_nxt);
        } else {
            if (active(t)) qk_tile(stage(t), s_now);
        }
        if (active(t)) {
            float alpha[NQ];
            bool rescale = false;
            if ((t + 1) * BN > wave_lim_min)
                softmax_tile(std::true_type{}, s_now, t, alpha, rescale);
            else
                softmax_tile(std::false_type{}, s_now, t, alpha, rescale);
            // O *= alpha after the masked / unmasked paths join: one place that
            // changes O outside the products keeps O in fixed registers
            if (rescale) {
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
                    for (int db = 0; db < D / 32; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[gq][db][r] *= alpha[gq];
            }
            pv_tile(stage(t) + TILE_B);
        }
    };
    f32x16 s_a[BN / 32][NQ], s_b[BN / 32][NQ];
    const int first = min(P, ntiles);
    for (int t = 0; t < first; ++t) issue_tile(t);
    if constexpr (PIPE) {
        if (ntiles > 0) {
            wait_tiles(first - 1);
            barrier_nofence();
            if (active(0)) qk_tile(stage(0), s_a);
        }
    }
    for (int t = 0; t < ntiles; t += 2) {
        step(t, s_a, s_b);
        if (t + 1 < ntiles) step(t + 1, s_b, s_a);
    }
    __syncthreads();  // all DMA landed (last wait was vmcnt(0)) and all reads done

    // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2 -------------------
    T* Os = reinterpret_cast<T*>(smem) + wave * 32 * NQ * OROW;
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        const float lt = l_run[gq] + swap_halves(l_run[gq]);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int qi = qw0 + gq * 32 + n32;
        if (hh == 0 && p.lse != nullptr && qi < p.Sq)
            p.lse[((int64_t)b * p.H + h) * p.Sq + qi] = lt > 0.f ? (m_run[gq] + log2f(lt)) * kLn2 : kNegInf;
        T* orow = Os + (gq * 32 + n32) * OROW;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = db * 32 + 8 * jj + 4 * hh;
                const f32x16& ov = oacc[gq][db];
                const u32x2 pk2 = {pack2<Tag>(ov[4 * jj] * inv, ov[4 * jj + 1] * inv),
                                   pack2<Tag>(ov[4 * jj + 2] * inv, ov[4 * jj + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + d0) = pk2;
            }
    }
    __syncthreads();
    for (int cidx = lane; cidx < 32 * NQ * CPR; cidx += 64) {
        const int row = cidx / CPR, cc = cidx - row * CPR;
        const int qi = qw0 + row;
        if (qi < p.Sq)
            *reinterpret_cast<u32x4*>(op + (int64_t)qi * p.sq.s + cc * 8) =
                *reinterpret_cast<const u32x4*>(Os + row * OROW + cc * 8);
    }
}

template <typename Tag, int D, int NQ, int BN, int NST, bool PIPE>
hipError_t launch16(const FwdArgs& a, hipStream_t stream) {
    constexpr int BM = 4 * 32 * NQ;
    Prefill16Params p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.kv_len = a.kv_len;
    p.sq = make_strides(a.layout, a.H, a.Sq, a.d);
    p.sk = make_strides(a.layout, a.H, a.Sk, a.d);
    p.B = a.B;
    p.H = a.H;
    p.Sq = a.Sq;
    p.Sk = a.Sk;
    p.c = a.scale * kLog2e;
    p.causal = a.causal ? 1 : 0;
    p.n_qtiles = (a.Sq + BM - 1) / BM;
    const int64_t grid = (int64_t)p.n_qtiles * a.B * a.H;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_prefill16_kernel<Tag, D, NQ, BN, NST, PIPE>), dim3((unsigned)grid), dim3(256), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t run_prefill16(const FwdArgs& a, hipStream_t stream) {
    if (a.dtype == 2)
        return a.d == 64 ? launch16<BF16, 64, 1, 64, 4, true>(a, stream)
                         : launch16<BF16, 128, 1, 32, 4, true>(a, stream);
    return a.d == 64 ? launch16<F16, 64, 1, 64, 4, true>(a, stream)
                     : launch16<F16, 128, 1, 32, 4, true>(a, stream);
}

}  // namespace attn
