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
//   * 4 waves per workgroup, each owning 32*NQ query rows (KSPLIT = 1), or 8
//     waves in two groups that each take half of every key tile (KSPLIT = 2,
//     see the ping-pong loop below).
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
//   * The running max serves as a reference: a tile's probabilities are taken
//     against it directly, and the exact tile max (with the rescale of l and
//     O) is computed only on a row's first tile or when the tile's row sum
//     shows the reference fell far behind. The result is the same up to
//     rounding because m, l and O always share one m.
//   * Workgroups of one head stay on one XCD (its L2 then serves every re-read
//     of that head's K/V); causal tiles start longest-first.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();
// A tile whose probabilities against the reference max sum to more than this
// (per lane, or are not finite) takes the exact-max path.
constexpr float kRefGuard = 4294967296.0f;  // 2^32

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

// KSPLIT = 1: 4 waves, wave w owns queries [32*NQ*w, +32*NQ) of the tile
//   and every key of every key tile.
// KSPLIT = 2: 8 waves; wave w owns queries [32*NQ*(w%4), +32*NQ) and the key
//   half (w/4) of every key tile, so each key/value operand read from LDS
//   feeds twice as many products per query row; the two halves' (m, l, O)
//   are merged through LDS after the key loop.
template <typename Tag, int D, int NQ, int BN, int NST, bool PIPE, int KSPLIT>
__global__ __launch_bounds__(256 * KSPLIT, 2 / KSPLIT) void fwd_prefill16_kernel(Prefill16Params p) {
    constexpr int NT = 256 * KSPLIT;               // threads
    constexpr int NW = 4 * KSPLIT;                 // waves
    constexpr int BM = 4 * 32 * NQ;                // query rows per workgroup
    constexpr int KBW = BN / 32 / KSPLIT;          // 32-key blocks per wave and tile
    constexpr int RB = D * 2;                      // bytes per K/V row
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int TILE_B = BN * RB;
    constexpr int STAGE_B = 2 * TILE_B;            // K tile, then V tile
    constexpr int DMA1 = TILE_B / 16 / NT;         // DMA loads per thread, tensor and tile
    constexpr int DPT = 2 * DMA1;                  // ... for K and V
    constexpr int P = NST - 1;                     // tiles in flight ahead
    constexpr int OROW = D + 8;                    // output staging row (elements)
    constexpr int OUT_B = 4 * 32 * NQ * OROW * 2;
    constexpr int MRG_W = (NQ * (D / 32) * 16 + 2 * NQ) * 64 * 4;  // one wave's (O, m, l) in fp32
    constexpr int MRG_B = KSPLIT == 2 ? 4 * MRG_W : 0;
    constexpr int LDS_A = NST * STAGE_B > OUT_B ? NST * STAGE_B : OUT_B;
    constexpr int LDS_B = LDS_A > MRG_B ? LDS_A : MRG_B;
    static_assert(KBW >= 1 && BN % (32 * KSPLIT) == 0, "key tile must split over the wave groups");
    static_assert(DMA1 >= 1 && TILE_B % (16 * NT) == 0, "tile must split over the lanes");
    static_assert(P >= (PIPE ? 2 : 1), "pipelining needs a deeper ring");
    static_assert(P * DPT < 64, "vmcnt range");
    using T = uint16_t;
    using SAcc = f32x16[KBW][NQ];

    __shared__ __align__(16) unsigned char smem[LDS_B];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave & 3;                // query group of this wave
    const int kh = wave >> 2;               // key half of this wave (KSPLIT = 2)
    const int kb0 = kh * KBW;               // first 32-key block of this wave in a tile
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

    const int qw0 = q0 + wq * 32 * NQ;  // first query row of this wave
    const bool wave_active = qw0 < p.Sq;
    const int wave_kend = p.causal ? min(nb, min(qw0 + 32 * NQ, p.Sq)) : nb;
    const int wave_lim_min = p.causal ? min(nb, qw0 + 1) : nb;  // keys past this need masks
    // first key of this wave's part of `tile`
    auto wkey0 = [&](int tile) { return tile * BN + kb0 * 32; };
    auto active = [&](int tile) { return wave_active && wkey0(tile) < wave_kend; };

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
    // Thread-slot i*NT + tid of the tile is the 16-byte chunk (row, pc); it
    // holds the logical chunk pc ^ swz(row) of key row `row`. Rows at or past
    // the valid length reread the last valid row (finite, masked later). The
    // per-thread offsets do not depend on the tile and are computed once.
    int64_t koff[DMA1], voff[DMA1];
#pragma unroll
    for (int i = 0; i < DMA1; ++i) {
        const int slot = i * NT + tid;
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
                dma16(kt + koff[i], st + i * NT * 16);
                dma16(vt + voff[i], st + i * NT * 16 + TILE_B);
            }
        } else {
#pragma unroll
            for (int i = 0; i < DMA1; ++i) {
                const int slot = i * NT + tid;
                const int row = slot / CPR, pc = slot - row * CPR;
                const int64_t key = min(key0 + row, nb - 1);
                dma16(kp + key * p.sk.s + (pc ^ swz_k<D>(row)) * 8, st + i * NT * 16);
                dma16(vp + key * p.sk.s + (pc ^ swz_v<D>(row)) * 8, st + i * NT * 16 + TILE_B);
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
    // A operand of S^T for key block kb (of the tile), K-step s
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

    auto qk_tile = [&](const unsigned char* kt, SAcc& sacc) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][gq][r] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) {
                const u32x4 a = k_operand(kt, kb0 + kb, s);
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) sacc[kb][gq] = mfma16<Tag>(a, qop[gq][s], sacc[kb][gq]);
            }
        }
    };

    // pq[gq][kb][u]: B operand of the (kb, u) product, the probabilities of
    // result registers 8u .. 8u+7 rounded and packed in pairs
    u32x4 pq[NQ][KBW][2];
    // Softmax of one tile against a reference max m_run (log2 units): the
    // probabilities are exp2(s c - m_run), rounded and packed for the second
    // product, and summed. The exact row max is only taken when a row has no
    // reference yet (its first tile) or when the tile's probabilities show the
    // reference fell far behind (a probability above 2^32, or infinite): then
    // m_run moves to the exact running max, l and O are rescaled by
    // exp2(m_old - m_new) (O after the caller's join, through `rescale`), and
    // the tile is redone. Any reference gives the same softmax; this one keeps
    // every probability below 2^32 while skipping the max on almost all tiles.
    auto softmax_tile = [&](auto masked_tag, SAcc& sacc, int tile, float (&alpha_out)[NQ], bool& rescale) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
            if constexpr (MASKED) {
                const int qi = qw0 + gq * 32 + n32;
                const int lim = p.causal ? min(nb, qi + 1) : nb;
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (wkey0(tile) + kb * 32 + blk_row(r, hh) >= lim) sacc[kb][gq][r] = kNegInf;
            }
            // probabilities against reference m (pack + partial row sum)
            auto exps = [&](float m) -> float {
                const float m_use = (m == kNegInf) ? 0.f : m;
                float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb)
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
                return (rs[0] + rs[1]) + (rs[2] + rs[3]);
            };
            alpha_out[gq] = 1.f;
            float rs_tile = 0.f;
            // at most two passes: the second only after the reference moved
            for (int pass = 0; pass < 2; ++pass) {
                rs_tile = exps(m_run[gq]);
                if (!__any(m_run[gq] == kNegInf || !(rs_tile <= kRefGuard))) break;
                // row max: four independent max3 chains, then the other lane half
                float mq[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
                for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; r += 4) {
                        const int ch = (kb * 4 + r / 4) & 3;
                        mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r], sacc[kb][gq][r + 1]));
                        mq[ch] = fmaxf(mq[ch], fmaxf(sacc[kb][gq][r + 2], sacc[kb][gq][r + 3]));
                    }
                float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
                mx = fmaxf(mx, swap_halves(mx));
                const float mxs = (MASKED && mx == kNegInf) ? kNegInf : mx * c;
                const float m_new = fmaxf(m_run[gq], mxs);
                const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[gq] - m_new);
                m_run[gq] = m_new;
                l_run[gq] *= alpha;
                alpha_out[gq] *= alpha;
                rescale = true;
                if (m_new == kNegInf) break;  // every key of the row masked so far: p = 0
            }
            l_run[gq] += rs_tile;
        }
    };

    auto pv_tile = [&](const unsigned char* vt) {
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const u32x4 a = v_operand(vt, kb0 + kb, u, db);
#pragma unroll
                    for (int gq = 0; gq < NQ; ++gq) oacc[gq][db] = mfma16<Tag>(a, pq[gq][kb][u], oacc[gq][db]);
                }
    };

    // softmax of tile t with the lazy rescale of O (applied after the masked /
    // unmasked paths join: one place that changes O outside the products
    // keeps O in fixed registers)
    auto softmax_step = [&](int t, SAcc& s_now) {
        float alpha[NQ];
        bool rescale = false;
        if (wkey0(t) + KBW * 32 > wave_lim_min)
            softmax_tile(std::true_type{}, s_now, t, alpha, rescale);
        else
            softmax_tile(std::false_type{}, s_now, t, alpha, rescale);
        if (rescale) {
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[gq][db][r] *= alpha[gq];
        }
    };

    if constexpr (KSPLIT == 2) {
        // ---- ping-pong key loop --------------------------------------------------
        // Per wave: M(t) = {O += P(t-1) V(t-1); S(t) = K(t) Q^T} on the matrix
        // cores, then V(t) = softmax of S(t) on the vector units. Both wave
        // groups run the same loop, [barrier] M(i) [barrier] V(i), but group 1
        // passes one extra barrier first (and group 0 one extra last), so group 1
        // runs half an iteration behind: on every SIMD one wave issues products
        // (at raised priority) while the other computes its softmax. Counting
        // workgroup barriers g = 0, 1, ...: group 0 runs M(i) after g = 2i,
        // group 1 after g = 2i+1. Tile t sits in stage t % 4: every wave waits
        // for its own part of it before g = 2t, and it is issued after
        // g = 2t-4, once both groups have finished M(t-3), the last reader of
        // tile t-4 in that stage.
        static_assert(NST == 4, "the ping-pong ring has four stages");
        auto wait_tile = [&](int t) {  // tiles issued after t by now: t+1 at most
            if (t + 1 < ntiles) wait_vmcnt<DPT>(); else wait_vmcnt<0>();
        };
        auto sync = [&]() {
            __builtin_amdgcn_sched_barrier(0);
            barrier_nofence();
            __builtin_amdgcn_sched_barrier(0);
        };
        for (int t = 0; t < min(2, ntiles); ++t) issue_tile(t);
        if (kh == 1) {  // g = 0
            if (ntiles > 0) wait_tile(0);
            sync();
            if (2 < ntiles) issue_tile(2);
        }
        for (int i = 0; i <= ntiles; ++i) {
            if (kh == 0 && i < ntiles) wait_tile(i);
            sync();  // group 0: g = 2i, group 1: g = 2i+1
            if (kh == 0 && i + 2 < ntiles) issue_tile(i + 2);
            SAcc s_cur;
            __builtin_amdgcn_s_setprio(1);
            if (i >= 1 && active(i - 1)) pv_tile(stage(i - 1) + TILE_B);
            if (i < ntiles && active(i)) qk_tile(stage(i), s_cur);
            __builtin_amdgcn_s_setprio(0);
            if (kh == 1 && i + 1 < ntiles) wait_tile(i + 1);
            sync();  // group 0: g = 2i+1, group 1: g = 2i+2
            if (kh == 1 && i + 3 < ntiles) issue_tile(i + 3);
            if (i < ntiles && active(i)) softmax_step(i, s_cur);
        }
        if (kh == 0) sync();  // g = 2*ntiles + 2
    } else {
        // ---- key loop over the DMA ring ---------------------------------------------
        // Unrolled by two so the score registers of tiles t and t+1 alternate
        // between two fixed sets instead of being copied.
        constexpr int AHEAD = PIPE ? 1 : 0;  // tiles needed beyond the one softmaxed
        auto step = [&](int t, SAcc& s_now, SAcc& s_nxt) {
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
                softmax_step(t, s_now);
                pv_tile(stage(t) + TILE_B);
            }
        };
        SAcc s_a, s_b;
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
    }
    __syncthreads();  // all DMA landed (last wait was vmcnt(0)) and all reads done

    // ---- merge the two key halves (KSPLIT = 2) ------------------------------
    // Lane (n32, h) of waves w and w+4 holds the same queries and the same
    // rows of O^T over disjoint keys: O = O_a 2^(m_a - m) + O_b 2^(m_b - m).
    if constexpr (KSPLIT == 2) {
        float* mrg = reinterpret_cast<float*>(smem) + wq * (MRG_W / 4);
        if (kh == 1) {
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mrg[((gq * (D / 32) + db) * 16 + r) * 64 + lane] = oacc[gq][db][r];
                mrg[(NQ * (D / 32) * 16 + 2 * gq) * 64 + lane] = m_run[gq];
                mrg[(NQ * (D / 32) * 16 + 2 * gq + 1) * 64 + lane] = l_run[gq];
            }
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
                const float mb = mrg[(NQ * (D / 32) * 16 + 2 * gq) * 64 + lane];
                const float lb = mrg[(NQ * (D / 32) * 16 + 2 * gq + 1) * 64 + lane];
                const float mm = fmaxf(m_run[gq], mb);
                const float mu = (mm == kNegInf) ? 0.f : mm;
                const float wa = fast_exp2(m_run[gq] - mu), wb = fast_exp2(mb - mu);
                m_run[gq] = mm;
                l_run[gq] = l_run[gq] * wa + lb * wb;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        oacc[gq][db][r] = oacc[gq][db][r] * wa + mrg[((gq * (D / 32) + db) * 16 + r) * 64 + lane] * wb;
            }
        }
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2 -------------------
    if (kh == 0) {
        T* Os = reinterpret_cast<T*>(smem) + wq * 32 * NQ * OROW;
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
    }
    __syncthreads();
    if (kh == 0) {
        const T* Os = reinterpret_cast<const T*>(smem) + wq * 32 * NQ * OROW;
        for (int cidx = lane; cidx < 32 * NQ * CPR; cidx += 64) {
            const int row = cidx / CPR, cc = cidx - row * CPR;
            const int qi = qw0 + row;
            if (qi < p.Sq)
                *reinterpret_cast<u32x4*>(op + (int64_t)qi * p.sq.s + cc * 8) =
                    *reinterpret_cast<const u32x4*>(Os + row * OROW + cc * 8);
        }
    }
}

template <typename Tag, int D, int NQ, int BN, int NST, bool PIPE, int KSPLIT>
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
    hipLaunchKernelGGL((fwd_prefill16_kernel<Tag, D, NQ, BN, NST, PIPE, KSPLIT>), dim3((unsigned)grid), dim3(256 * KSPLIT), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

// Kernel choice (measured on MI355X): head size 64 over long key ranges uses
// the 8-wave ping-pong kernel (half the LDS operand traffic per product and
// products of one group overlapping the other group's softmax); short key
// ranges, where its pipeline fill and final merge do not pay off, and head
// size 128 use the 4-wave pipelined kernel.
constexpr int kPingPongMinKeys = 2048;

hipError_t run_prefill16(const FwdArgs& a, hipStream_t stream) {
    const bool pp = a.d == 64 && a.Sk >= kPingPongMinKeys;
    if (a.dtype == 2) {
        if (a.d == 128) return launch16<BF16, 128, 1, 32, 4, true, 1>(a, stream);
        return pp ? launch16<BF16, 64, 2, 64, 4, true, 2>(a, stream) : launch16<BF16, 64, 1, 64, 4, true, 1>(a, stream);
    }
    if (a.d == 128) return launch16<F16, 128, 1, 32, 4, true, 1>(a, stream);
    return pp ? launch16<F16, 64, 2, 64, 4, true, 2>(a, stream) : launch16<F16, 64, 1, 64, 4, true, 1>(a, stream);
}

}  // namespace attn
