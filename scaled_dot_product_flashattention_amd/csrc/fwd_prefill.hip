// Fused attention forward for fp32 inputs: one kernel, scores and
// probabilities stay on chip (16-bit inputs run fwd_prefill16.hip).
//
// Method (chapter "2. 自注意力机制算子…以及FlashAttention优化", §2.6, and the
// section "FlashAttention 分块计算原理与浏览器适配" of the WebGPU page): the
// queries of one head are cut into tiles of BM rows, the keys/values into
// tiles of BN rows. A workgroup owns one query tile, streams every key/value
// tile it needs through LDS, and keeps per query row a running maximum m and a
// running sum l; when a new tile raises m, the sum and the partial output are
// first multiplied by exp(m_old - m_new). The output is divided by l once, at
// the end.
//
// Mapping to gfx950:
//   * 4 waves per workgroup, each owning 32*NQ query rows; BM = 128*NQ.
//   * Scores are computed transposed, S^T = K Q^T, with 32x32x2 fp32
//     matrix-core blocks: a lane then owns one query (its column) and 32 of the 64 keys
//     of a tile (its rows), so the row max and row sum are in-lane except for
//     one exchange between the two lane halves.
//   * The output is kept transposed too, O^T += V^T P^T: the probabilities
//     feed the second product straight from the score registers, and the
//     rescale by exp(m_old - m_new) touches only the lane's own query.
//   * K tiles sit in LDS row-major; V tiles are transposed while being stored
//     to LDS so both operands are read as contiguous vectors. Both are double
//     buffered: tile t+1 is fetched into registers while tile t is computed.
//   * Workgroups of one head are kept on one XCD (its L2 then serves every
//     re-read of that head's K/V); causal tiles are started longest-first.
//   * Exponentials are base 2 with scale*log2(e) folded into one FMA.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();
// The running max moves only when a tile's max exceeds it by more than this
// (base-2 units): probabilities then stay below 2^8 and most tiles skip the
// rescale of the partial output.
constexpr float kLazyRescale = 8.0f;

struct PrefillParams {
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
    int remap;  // grid size is a multiple of 8: group each head's tiles on one XCD
};

template <typename Tag, int D, int NQ>
struct PrefillCfg {
    static constexpr int NW = 4;                 // waves per workgroup
    static constexpr int BM = NW * 32 * NQ;      // query rows per workgroup
    static constexpr int BN = 64;                // keys per tile
    static constexpr int ES = Tag::bytes;        // element bytes
    static constexpr int KROW = D + 16 / ES;     // LDS K row, padded by 16 B
    static constexpr int VROW = BN + 8 / ES;     // LDS V^T row, padded by 8 B
    static constexpr int K_ELEMS = BN * KROW;
    static constexpr int V_ELEMS = D * VROW;
    static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * ES;
    static constexpr int OROW = D + 16 / ES;     // output staging row
    static constexpr int OUT_BYTES = NW * 32 * NQ * OROW * ES;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES > OUT_BYTES ? 2 * STAGE_BYTES : OUT_BYTES;
    static constexpr int EPC = 16 / ES;          // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;          // 16-byte chunks per row
    static constexpr int KCH = BN * CPR / 256;   // K chunks per thread and tile
    static_assert(BN * CPR % 256 == 0, "tile must split evenly over 256 threads");
};

template <typename Tag, int D, int NQ, bool PIPE>
__global__ __launch_bounds__(256, 2) void fwd_prefill_kernel(PrefillParams p) {
    using C = PrefillCfg<Tag, D, NQ>;
    using T = typename Tag::storage;
    constexpr int BN = C::BN;
    static_assert(C::ES == 4, "fp32 inputs only");

    __shared__ __align__(16) unsigned char smem[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const int q0 = qt * C::BM;
    const int q_end = min(q0 + C::BM, p.Sq);
    const int kend = p.causal ? min(nb, q_end) : nb;  // keys any row of the tile can see
    const int ntiles = (kend + BN - 1) / BN;

    const T* qp = static_cast<const T*>(p.q) + p.sq.head(b, h);
    const T* kp = static_cast<const T*>(p.k) + p.sk.head(b, h);
    const T* vp = static_cast<const T*>(p.v) + p.sk.head(b, h);
    T* op = static_cast<T*>(p.o) + p.sq.head(b, h);

    const int qw0 = q0 + wave * 32 * NQ;  // first query row of this wave
    const bool wave_active = qw0 < p.Sq;
    const int wave_kend = p.causal ? min(nb, min(qw0 + 32 * NQ, p.Sq)) : nb;
    const int wave_lim_min = p.causal ? min(nb, qw0 + 1) : nb;  // tiles past this need masks

    // ---- Q operands, held in registers for the whole key loop -------------
    // B operand of S^T = K Q^T: K-step s holds q[row][2s + h].
    constexpr int QSTEPS = D / 2;
    float qop[NQ][QSTEPS];
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        const int qi = qw0 + gq * 32 + n32;
        const bool ok = qi < p.Sq;
        const T* row = qp + (int64_t)(ok ? qi : 0) * p.sq.s;
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) qop[gq][s] = ok ? row[2 * s + hh] : 0.f;
    }

    // ---- global -> register -> LDS staging of one K/V tile -----------------
    // K and V: 16-byte chunks, consecutive threads along a row (coalesced);
    // V is transposed element by element when stored to LDS.
    constexpr int VCH = BN * C::CPR / 256;
    static_assert(VCH >= 1, "V tile must cover all threads");
    u32x4 kreg[C::KCH];
    u32x4 vreg[VCH];

    auto load_k = [&](int t) {
        const int key0 = t * BN;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < C::KCH; ++c) {
            const int idx = tid + c * 256;
            const int row = idx / C::CPR, cc = idx - row * C::CPR;
            const int key = key0 + row;
            kreg[c] = key < nb ? *reinterpret_cast<const u32x4*>(kp + (int64_t)key * p.sk.s + cc * C::EPC) : z;
        }
    };
    auto load_v = [&](int t) {
        const int key0 = t * BN;
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < VCH; ++c) {
            const int idx = tid + c * 256;
            const int row = idx / C::CPR, cc = idx - row * C::CPR;
            const int key = key0 + row;
            vreg[c] = key < nb ? *reinterpret_cast<const u32x4*>(vp + (int64_t)key * p.sk.s + cc * C::EPC) : z;
        }
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

    auto k_lds = [&](int tile) {
        return reinterpret_cast<const T*>(smem + (tile & 1) * C::STAGE_BYTES);
    };
    auto v_lds = [&](int tile) { return k_lds(tile) + C::K_ELEMS; };
    auto active = [&](int tile) { return wave_active && tile * BN < wave_kend; };

    // -- S^T = K Q^T for one key tile (keys x queries, BN/32 blocks of 32) -----
    auto qk_tile = [&](const T* Ks, f32x16 (&sacc)[BN / 32][NQ]) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[kb][gq][r] = 0.f;
#pragma unroll
        for (int s = 0; s < QSTEPS; ++s) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb) {
                const float a = Ks[(kb * 32 + n32) * C::KROW + 2 * s + hh];
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) sacc[kb][gq] = mfma_f32(a, qop[gq][s], sacc[kb][gq]);
            }
        }
    };

    // -- online softmax of one tile: running max (moved lazily), probabilities
    //    in place of the scores, running sum ----------------------------------
    auto softmax_tile = [&](auto masked_tag, f32x16 (&sacc)[BN / 32][NQ], int tile) {
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
            // row max: four independent max3 chains, then the other lane half
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
            // move the reference max only when the tile max exceeds it by more
            // than kLazyRescale (log2 units); the wave decides together.
            if (__any(mxs > m_run[gq] + kLazyRescale)) {
                const float m_new = fmaxf(m_run[gq], mxs);
                const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run[gq] - m_new);
                m_run[gq] = m_new;
                l_run[gq] *= alpha;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[gq][db][r] *= alpha;
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
                    sacc[kb][gq][r] = p0;
                    sacc[kb][gq][r + 1] = p1;
                    rs[(r / 2) & 3] += p0 + p1;
                }
            l_run[gq] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        }
    };

    // -- O^T += V^T P^T ----------------------------------------------------------
    auto pv_tile = [&](const T* Vt, f32x16 (&sacc)[BN / 32][NQ]) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const float a = Vt[(db * 32 + n32) * C::VROW + kb * 32 + blk_row(r, hh)];
#pragma unroll
                    for (int gq = 0; gq < NQ; ++gq) oacc[gq][db] = mfma_f32(a, sacc[kb][gq][r], oacc[gq][db]);
                }
            }
        }
    };

    // ---- key loop ----------------------------------------------------------------
    // PIPE: LDS holds K of tile t+1 and V of tile t while tile t is processed,
    // so the scores of tile t+1 are issued before the softmax of tile t (K is
    // staged two tiles ahead, V one). Without PIPE both are staged one ahead
    // and tile t's scores are computed at the start of its iteration. K_t and
    // V_t live in LDS stage t & 1.
    constexpr int KAHEAD = PIPE ? 2 : 1;
    auto store_k = [&](int tile) {
        T* Ks = reinterpret_cast<T*>(smem + (tile & 1) * C::STAGE_BYTES);
#pragma unroll
        for (int cc2 = 0; cc2 < C::KCH; ++cc2) {
            const int idx = tid + cc2 * 256;
            const int row = idx / C::CPR, cc = idx - row * C::CPR;
            *reinterpret_cast<u32x4*>(Ks + row * C::KROW + cc * C::EPC) = kreg[cc2];
        }
    };
    auto store_v = [&](int tile) {
        T* Vt = reinterpret_cast<T*>(smem + (tile & 1) * C::STAGE_BYTES) + C::K_ELEMS;
#pragma unroll
        for (int c2 = 0; c2 < VCH; ++c2) {
            const int idx = tid + c2 * 256;
            const int row = idx / C::CPR, cc = idx - row * C::CPR;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                reinterpret_cast<uint32_t*>(Vt)[(cc * 4 + e) * C::VROW + row] = vreg[c2][e];
        }
    };

    f32x16 s_cur[BN / 32][NQ];
    if (ntiles > 0) {
        load_v(0);
        store_v(0);
#pragma unroll
        for (int a = 0; a < KAHEAD; ++a)
            if (a < ntiles) {
                load_k(a);
                store_k(a);
            }
    }
    __syncthreads();
    if constexpr (PIPE) {
        if (ntiles > 0 && active(0)) qk_tile(k_lds(0), s_cur);
        __syncthreads();  // every wave has read K_0 before its stage is reused
    }

    for (int t = 0; t < ntiles; ++t) {
        if (t + KAHEAD < ntiles) load_k(t + KAHEAD);
        if (t + 1 < ntiles) load_v(t + 1);

        f32x16 s_next[BN / 32][NQ];
        if constexpr (PIPE) {
            if (t + 1 < ntiles && active(t + 1)) qk_tile(k_lds(t + 1), s_next);
        } else {
            if (active(t)) qk_tile(k_lds(t), s_cur);
        }

        if (active(t)) {
            if ((t + 1) * BN > wave_lim_min)
                softmax_tile(std::true_type{}, s_cur, t);
            else
                softmax_tile(std::false_type{}, s_cur, t);
            pv_tile(v_lds(t), s_cur);
        }
        if constexpr (PIPE) {
#pragma unroll
            for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
                for (int gq = 0; gq < NQ; ++gq) s_cur[kb][gq] = s_next[kb][gq];
        }

        if (t + KAHEAD < ntiles) store_k(t + KAHEAD);
        if (t + 1 < ntiles) store_v(t + 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2 -------------------
    T* Os = reinterpret_cast<T*>(smem) + wave * 32 * NQ * C::OROW;
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        const float lt = l_run[gq] + __shfl_xor(l_run[gq], 32);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int qi = qw0 + gq * 32 + n32;
        if (hh == 0 && p.lse != nullptr && qi < p.Sq)
            p.lse[((int64_t)b * p.H + h) * p.Sq + qi] = lt > 0.f ? (m_run[gq] + log2f(lt)) * kLn2 : kNegInf;
        T* orow = Os + (gq * 32 + n32) * C::OROW;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d0 = db * 32 + 8 * jj + 4 * hh;
                const f32x16& ov = oacc[gq][db];
                const f32x4 o4 = {ov[4 * jj] * inv, ov[4 * jj + 1] * inv, ov[4 * jj + 2] * inv,
                                  ov[4 * jj + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + d0) = o4;
            }
    }
    __syncthreads();
    // coalesced copy of the wave's rows to global memory
    for (int cidx = lane; cidx < 32 * NQ * C::CPR; cidx += 64) {
        const int row = cidx / C::CPR, cc = cidx - row * C::CPR;
        const int qi = qw0 + row;
        if (qi < p.Sq)
            *reinterpret_cast<u32x4*>(op + (int64_t)qi * p.sq.s + cc * C::EPC) =
                *reinterpret_cast<const u32x4*>(Os + row * C::OROW + cc * C::EPC);
    }
}

template <typename Tag, int D, int NQ, bool PIPE>
hipError_t launch_prefill(const FwdArgs& a, hipStream_t stream) {
    using C = PrefillCfg<Tag, D, NQ>;
    PrefillParams p;
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
    p.n_qtiles = (a.Sq + C::BM - 1) / C::BM;
    const int64_t grid = (int64_t)p.n_qtiles * a.B * a.H;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_prefill_kernel<Tag, D, NQ, PIPE>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t run_prefill(const FwdArgs& a, hipStream_t stream) {
    if (a.dtype != 0) return run_prefill16(a, stream);
    if (a.tile > 0 || a.n_split > 1) return hipErrorInvalidValue;  // fp32: one variant, no key splits
    return a.d == 64 ? launch_prefill<F32, 64, 1, false>(a, stream) : launch_prefill<F32, 128, 1, false>(a, stream);
}

// fp32 inputs have a single tile variant per head size.
int prefill_tile_count(int d, int dtype) { return dtype == 0 ? 1 : prefill16_tile_count(d); }

bool prefill_tile_info(int d, int dtype, int tile, TileInfo* out) {
    if (dtype != 0) return prefill16_tile_info(d, tile, out);
    if (tile != 0 || (d != 64 && d != 128)) return false;
    out->rows = PrefillCfg<F32, 64, 1>::BM;
    out->keys = PrefillCfg<F32, 64, 1>::BN;
    out->waves = PrefillCfg<F32, 64, 1>::NW;
    out->stages = 2;
    out->lds_bytes = d == 64 ? PrefillCfg<F32, 64, 1>::LDS_BYTES : PrefillCfg<F32, 128, 1>::LDS_BYTES;
    return true;
}

int prefill_tile_choice(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int n_split) {
    return dtype == 0 ? 0 : prefill16_tile_choice(B, H, Sq, Sk, d, causal, n_split);
}

}  // namespace attn
