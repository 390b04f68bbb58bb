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
//   * Scores are computed transposed, S^T = K Q^T, on 32x32x16 matrix-core
//     blocks: a lane owns one query (its column) and half the keys of each
//     32-key block (its rows), so a row max is in-lane but for one exchange
//     between the two lane halves (v_permlane32_swap).
//   * The output is kept transposed too, O^T += V^T P^T: probabilities feed
//     the second product straight from the score registers (rounded and
//     packed in pairs), and a rescale touches only the lane's own query.
//   * Row sums on the matrix core: each 16-key block of rounded
//     probabilities, as it stands for the output product, is also the B
//     operand of one 16x16x32 product with a fixed 0/1 selector as A. The
//     selector routes the 16 keys of query q into the result row that lane q
//     (and lane q + 32) holds in its first register, so every lane keeps the
//     whole-row sum of its own query. This replaces 8 pairwise adds per block
//     on the vector unit, which sets the pace of this loop, by one product
//     an eighth the size of the output products.
//   * Software pipeline inside each wave: while the vector unit computes the
//     softmax of key tile t, the same wave issues the matrix products of
//     P(t-1) V(t-1) and K(t+1) Q^T, one product between every few
//     probabilities. On gfx950 a wave's own vector instructions issue while
//     its matrix product runs. The probabilities themselves go in three
//     stages over consecutive product slots (scale and shift, exponential,
//     rounding), so no vector instruction waits on the one just before it.
//     Two wave groups in opposite, barrier-separated phases (one multiplying
//     while the other computes probabilities) were measured much slower, so
//     the overlap is arranged within the wave.
//   * K and V tiles travel global -> LDS by direct DMA loads
//     (global_load_lds_dwordx4) into an NST-stage ring, NST-2 tiles ahead of
//     the tile whose keys are multiplied (NST-3 for rings of 6 or more
//     stages, which pass one barrier per two tiles); no registers are spent
//     on staging. At head size 64 four waves issue them (with two key
//     halves, the waves of half 0, which run ahead of their SIMD partners).
//     Both sit in LDS row-major with their 16-byte chunks XOR-swizzled per
//     row so that the K operand reads (ds_read_b128) and the transposing V
//     operand reads (ds_read_b64_tr_b16) are free of bank conflicts; the K
//     tiles of every stage come first, then the V tiles, so that when each
//     tensor's ring fits 64 KiB every operand address is a per-lane base plus
//     an immediate offset (with the key loop unrolled over the stages).
//   * KSPLIT = 2: two groups of 4 waves take the two key halves of every
//     tile for the same queries (each key operand then feeds two query
//     blocks), and merge their (m, l, O) through LDS at the end. Their Q
//     rows are loaded once, into LDS, and read from there by both groups.
//   * The running max is a reference: it starts at the exact maximum of
//     each row over the wave's first key tile, and later probabilities are
//     taken against it directly; only the row sum is checked. The exact max
//     (with the rescale of l and O) is taken again only when a lane's sum
//     passes 2^32 (or a 16-bit probability overflows), i.e. when a later
//     tile's scores rise far above the first tile's. Any common reference
//     gives the same softmax; starting at a row's own maximum keeps its
//     largest probabilities at 1 or more, in the normal range of fp16.
//   * Workgroups of one head stay on one XCD (its L2 then serves every re-read
//     of that head's K/V); causal tiles start longest-first, across all the
//     heads of an XCD when their K/V are small enough to share its L2.
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr float kNegInf = -__builtin_inff();
// The reference max stays while every row's running sum is at most 2^32
// (bit pattern below). The reference starts at the row's maximum over its
// first tile, so each row's sum is at least 1 from then on and nothing of
// weight underflows.
constexpr uint32_t kSumHiBits = 0x4F800000u;  // 2^32

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int V> using int_c = std::integral_constant<int, V>;

// f(int_c<K>) for K = 0, 1, ... in order.
template <typename F, int... K>
__device__ __forceinline__ void for_each_stage(F&& f, std::integer_sequence<int, K...>) {
    (f(int_c<K>{}), ...);
}

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
    // causal mask with B*H a multiple of 8 (key ranges excluded) and the K/V
    // of one XCD's heads within kCausalMixBytes: those B*H/8 heads take
    // turns, query tile by query tile (0: head by head)
    int causal_heads;
    // key splits (SPLIT kernels): workgroup split s takes keys
    // [s * chunk, (s + 1) * chunk) and writes its (m, l, o) records to ws
    float* ws;
    int n_split;
    int chunk;
};

// LDS of one workgroup: the K/V ring (then, with two key halves, the staged
// Q rows when they fit beside it in 160 KiB), reused for the output staging
// rows (D + 8 elements per query) and, with two key halves, for the merge of
// the halves' (O, m, l) in fp32.
constexpr int lds_bytes16(int D, int NQ, int BN, int NST, int KSPLIT) {
    const int ring0 = NST * 2 * BN * D * 2;
    const int qb = 4 * 32 * NQ * D * 2;  // staged Q rows (two key halves)
    const int ring = ring0 + ((KSPLIT == 2 && ring0 + qb <= 160 * 1024) ? qb : 0);
    const int out = 4 * 32 * NQ * (D + 8) * 2;
    const int mrg = KSPLIT == 2 ? 8 * (NQ * (D / 64) * 16 + 2 * NQ) * 64 * 4 : 0;
    const int a = ring > out ? ring : out;
    return a > mrg ? a : mrg;
}

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

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit byte offset
// per lane: the per-load address arithmetic stays on the scalar unit.
__device__ __forceinline__ void dma16_sb(const void* base, uint32_t off, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds_addr) : "memory");
}

// Workgroup barrier without a memory fence: each wave has already waited for
// its own DMA loads; the empty asm statements keep the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// True where a running row sum (never negative) passed 2^32, is infinite (a
// 16-bit probability overflowed) or is not a number.
__device__ __forceinline__ bool sum_out_of_range(float l) {
    return __float_as_uint(l) > kSumHiBits;
}

// Template parameters:
//   D      head size (64 or 128)
//   NQ     32-query blocks per wave (BM = 128 * NQ queries per workgroup)
//   BN     keys per tile
//   NST    LDS ring stages (NST - 2 tiles in flight ahead)
//   KSPLIT 1: 4 waves, each over all keys of a tile; 2: 8 waves, wave w
//          takes key half w / 4 of every tile for the queries of wave w % 4
//   OCC    waves per SIMD the registers are sized for (two; three for a
//          lean tile whose workgroups share a compute unit three at a time)
//   SPLIT  each workgroup takes one range of p.chunk keys and, instead of
//          O and LSE, writes per query row the record (m, l, -, -, o[D]) of
//          its range: the reference max m (log2 units; -inf when l = 0), the
//          sum l against it and the unnormalised output o. The records of
//          the ranges of a row combine exactly by the block rule.
template <typename Tag, int D, int NQ, int BN, int NST, int KSPLIT, int OCC, bool SPLIT>
__global__ __launch_bounds__(256 * KSPLIT, OCC / KSPLIT) void fwd_prefill16_kernel(Prefill16Params p) {
    constexpr int KBW = BN / 32 / KSPLIT;          // 32-key blocks per wave and tile
    constexpr int RB = D * 2;                      // bytes per K/V row
    constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    constexpr int TILE_B = BN * RB;
    constexpr int STAGE_B = TILE_B;                // stage stride: K tiles of every stage, then V tiles
    constexpr int VOFF = NST * TILE_B;             // V tile of stage g at VOFF + g * TILE_B
    // At head size 64 with two key halves only the four waves of half 0
    // issue the DMA loads: they win issue arbitration against their SIMD
    // partners of half 1 and reach each barrier first, so the stall of
    // issuing (a wave waits while the CU's load queue drains) costs least
    // there. (At head size 128 the 5-stage variant then spilled registers
    // inside its key loop, so all eight waves issue there.)
    constexpr int NIW = D == 64 ? 4 : 4 * KSPLIT;  // waves that issue DMA loads
    constexpr int NIT = NIW * 64;
    constexpr int DMA1 = TILE_B / 16 / NIT;        // DMA loads per issuing thread, tensor and tile
    constexpr int DPT = 2 * DMA1;                  // ... for K and V
    // Rings of 6 or more stages take one barrier per two tiles (at even t),
    // which costs one stage of lookahead.
    constexpr bool BAR2 = NST >= 6;
    constexpr int P = BAR2 ? NST - 3 : NST - 2;    // tiles issued ahead
    constexpr int OROW = D + 8;                    // output staging row (elements)
    constexpr int MRG_W = (NQ * (D / 64) * 16 + 2 * NQ) * 64 * 4;  // half a wave's O, its (m, l), fp32
    constexpr int LDS_B = lds_bytes16(D, NQ, BN, NST, KSPLIT);
    constexpr int NPV = KBW * 2 * (D / 32) * NQ;   // products of P V per tile and wave
    constexpr int NQK = (D / 16) * KBW * NQ;       // products of K Q^T per tile and wave
    constexpr int NM = NPV + NQK;
    constexpr int NPAIR = NQ * KBW * 8;            // probability pairs per lane and tile
    static_assert(KBW >= 1 && BN % (32 * KSPLIT) == 0, "key tile must split over the wave groups");
    static_assert(DMA1 >= 1 && TILE_B % (16 * NIT) == 0, "tile must split over the lanes");
    static_assert(P >= 2, "the pipeline needs two tiles in flight");
    static_assert(!BAR2 || P >= 3, "tile t+2 must be issued before the barrier of t");
    static_assert((P - 2) * DPT < 64, "vmcnt range");
    using T = uint16_t;
    using SAcc = f32x16[KBW][NQ];
    using PAcc = u32x4[NQ][KBW][2];

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
    constexpr int BM = 4 * 32 * NQ;
    const int G = gridDim.x;
    const int g = blockIdx.x;
    int w = p.remap ? (g & 7) * (G >> 3) + (g >> 3) : g;
    if (p.causal_heads) {
        // XCD x (workgroups g = x mod 8) still takes the heads of its range,
        // but in the order (query tile, head): with the reversal below, the
        // longest tiles of all its heads go first. Head by head, a late
        // head's longest tile would start last and end the kernel.
        const int j = g >> 3;
        const int qrank = j / p.causal_heads;
        w = (g & 7) * (G >> 3) + (j - qrank * p.causal_heads) * p.n_qtiles + qrank;
    }
    // query tiles innermost: the tiles of one key range of a head run
    // together and share its K/V in L2
    int split = 0;
    if constexpr (SPLIT) {
        const int rest = w / p.n_qtiles;
        split = rest % p.n_split;
        w = (rest / p.n_split) * p.n_qtiles + (w - rest * p.n_qtiles);
    }
    const int bh = w / p.n_qtiles;
    int qt = w - bh * p.n_qtiles;
    if (p.causal) qt = p.n_qtiles - 1 - qt;  // longest causal tiles first
    const int b = bh / p.H;
    const int h = bh - b * p.H;

    const int q0 = qt * BM;
    const T* qp = static_cast<const T*>(p.q) + p.sq.head(b, h);
    const int qw0 = q0 + wq * 32 * NQ;  // first query row of this wave
    // ---- Q operands (B of S^T = K Q^T), in registers for the whole loop ----
    // K-step s holds q[row][16s + 8h .. +7]. Their loads go out first:
    // nothing in them waits for the per-batch key length, a load of its own
    // (the fence keeps the compiler from waiting for it earlier).
    u32x4 qop[NQ][D / 16];
    // With two key halves both waves of a query group need the same Q: the
    // first four waves load the workgroup's BM rows once, by DMA, into LDS
    // after the K/V ring (where they fit; else each wave loads its own), and
    // every wave reads its operands from there after the prologue's barrier.
    constexpr bool QLDS = KSPLIT == 2 && 2 * NST * TILE_B + BM * RB <= 160 * 1024;
    constexpr int QOFF = 2 * NST * TILE_B;  // LDS byte offset of the staged Q rows
    if constexpr (QLDS) {
        if (wave < 4) {
            const uint32_t st = __builtin_amdgcn_readfirstlane(
                (uint32_t)(uintptr_t)(lds_void*)smem + QOFF + wave * 1024);
#pragma unroll
            for (int i = 0; i < BM * CPR / 256; ++i) {
                const int slot = i * 256 + tid;
                const int row = slot / CPR, pc = slot - row * CPR;
                // rows past the last query reread it (finite; never stored)
                const int64_t qi = min(q0 + row, p.Sq - 1);
                dma16(qp + qi * p.sq.s + (pc ^ swz_k<D>(row)) * 8, st + i * 256 * 16);
            }
        }
    } else {
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
    }
    __builtin_amdgcn_sched_barrier(0);
    const int nb = clamp_len(p.kv_len, b, p.Sk);
    const int q_end = min(q0 + BM, p.Sq);
    const int kend = p.causal ? min(nb, q_end) : nb;  // keys any row of the tile can see
    const int key_lo = SPLIT ? split * p.chunk : 0;   // this workgroup's keys: [key_lo, key_hi)
    const int key_hi = SPLIT ? min(key_lo + p.chunk, kend) : kend;
    const int ntiles = key_hi > key_lo ? (key_hi - key_lo + BN - 1) / BN : 0;
    const int lim_hi = SPLIT ? key_hi : nb;  // keys from here on are masked for every row

    const T* kp = static_cast<const T*>(p.k) + p.sk.head(b, h);
    const T* vp = static_cast<const T*>(p.v) + p.sk.head(b, h);
    T* op = static_cast<T*>(p.o) + p.sq.head(b, h);

    // Waves past the last query row compute on zero queries and store nothing.
    const int wave_lim_min = p.causal ? min(lim_hi, qw0 + 1) : lim_hi;  // keys past this need masks
    // first key of this wave's part of `tile`
    auto wkey0 = [&](int tile) __attribute__((always_inline)) { return key_lo + tile * BN + kb0 * 32; };

    // ---- DMA of one K/V tile into LDS stage tile % NST ----------------------
    // Issuing-thread slot i*NIT + tid of the tile is the 16-byte chunk (row,
    // pc); it holds the logical chunk pc ^ swz(row) of key row `row`. Rows at
    // or past the valid length reread the last valid row (finite, masked
    // later). Pass i covers key rows [i RPP, (i+1) RPP); the swizzles repeat
    // every 16 rows, so a thread's offsets differ between passes by whole
    // rows, and the offsets of pass 0 are computed once.
    constexpr int RPP = NIT / CPR;
    static_assert(RPP % 16 == 0, "swizzle period must divide the rows per pass");
    // The loads of a whole tile take a wave-uniform 64-bit base in SGPRs and
    // a 32-bit byte offset per lane, so no vector instruction computes an
    // address. At head size 128 each pass has its own offset register; at
    // head size 64 one offset serves every pass and the pass's rows go into
    // the scalar base, which saves the registers whose spills (with a reload
    // whose wait drained the DMA queue) cost the eight-wave variant 2.5 %
    // (measured on gfx950; at head size 128 per-pass offsets were 1 % faster).
    constexpr bool DMA_ONE_OFF = D == 64;
    uint32_t kofb[DMA1], vofb[DMA1];
    {
        const int slot = tid & (NIT - 1);
        const int row = slot / CPR, pc = slot - row * CPR;
        const int64_t koff = row * p.sk.s + (pc ^ swz_k<D>(row)) * 8;
        const int64_t voff = row * p.sk.s + (pc ^ swz_v<D>(row)) * 8;
#pragma unroll
        for (int i = 0; i < DMA1; ++i) {
            kofb[i] = (uint32_t)((koff + (int64_t)i * RPP * p.sk.s) * 2);
            vofb[i] = (uint32_t)((voff + (int64_t)i * RPP * p.sk.s) * 2);
        }
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)smem;
    auto issue_tile = [&](int tile) __attribute__((always_inline)) {
        if (wave >= NIW) return;
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + (tile % NST) * STAGE_B + wave * 1024);
        const int key0 = key_lo + tile * BN;
        if (key0 + BN <= nb) {
            const T* kt = kp + key0 * p.sk.s;
            const T* vt = vp + key0 * p.sk.s;
#pragma unroll
            for (int i = 0; i < DMA1; ++i) {
                if constexpr (DMA_ONE_OFF) {
                    dma16_sb(kt + (int64_t)i * RPP * p.sk.s, kofb[0], st + i * NIT * 16);
                    dma16_sb(vt + (int64_t)i * RPP * p.sk.s, vofb[0], st + i * NIT * 16 + VOFF);
                } else {
                    dma16_sb(kt, kofb[i], st + i * NIT * 16);
                    dma16_sb(vt, vofb[i], st + i * NIT * 16 + VOFF);
                }
            }
        } else {
            // A partial last tile recomputes its addresses from the thread
            // index: the opaque copy keeps the compiler from hoisting them
            // out of the key loop into registers held for the whole loop.
            int tid_r = tid;
            asm volatile("" : "+v"(tid_r));
#pragma unroll
            for (int i = 0; i < DMA1; ++i) {
                const int slot = i * NIT + tid_r;
                const int row = slot / CPR, pc = slot - row * CPR;
                const int64_t key = min(key0 + row, nb - 1);
                dma16(kp + key * p.sk.s + (pc ^ swz_k<D>(row)) * 8, st + i * NIT * 16);
                dma16(vp + key * p.sk.s + (pc ^ swz_v<D>(row)) * 8, st + i * NIT * 16 + VOFF);
            }
        }
    };
    // Wait until this thread's DMA loads of `tile` have landed, given that
    // tiles up to `last_issued` (at most tile + P - 2) were issued after it.
    auto wait_tile = [&](int tile, int last_issued) __attribute__((always_inline)) {
        const int after = last_issued - tile;
        if constexpr (P - 2 >= 4) { if (after >= 4) { wait_vmcnt<((P - 2 >= 4) ? 4 * DPT : 0)>(); return; } }
        if constexpr (P - 2 >= 3) { if (after >= 3) { wait_vmcnt<((P - 2 >= 3) ? 3 * DPT : 0)>(); return; } }
        if constexpr (P - 2 >= 2) { if (after >= 2) { wait_vmcnt<((P - 2 >= 2) ? 2 * DPT : 0)>(); return; } }
        if constexpr (P - 2 >= 1) { if (after >= 1) { wait_vmcnt<((P - 2 >= 1) ? DPT : 0)>(); return; } }
        wait_vmcnt<0>();
    };

    // ---- operand reads ----------------------------------------------------------
    auto stage = [&](int tile) __attribute__((always_inline)) { return smem + (tile % NST) * STAGE_B; };
    // A operand of S^T for key block kb (of the tile), K-step s
    auto k_operand = [&](const unsigned char* kt, int kb, int s) __attribute__((always_inline)) -> u32x4 {
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
    auto v_operand = [&](const unsigned char* vt, int kb, int u, int db) __attribute__((always_inline)) -> u32x4 {
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
    // Operands are read LA product slots ahead of their first product: K
    // operand o (K-step o / KBW, key block o % KBW) feeds products
    // NPV + o*NQ .. +NQ-1 of an iteration, V operand o (key block, u, db in
    // that order) feeds products o*NQ .. +NQ-1. V operands due in the first
    // LA slots are read at the end of the previous iteration.
    constexpr int NV = KBW * 2 * (D / 32);
    constexpr int NK = KBW * (D / 16);
    constexpr int LA = 4;
    u32x4 kop[NK];
    u32x4 vop[NV];
    auto read_kop = [&](int o, const unsigned char* kt) __attribute__((always_inline)) {
        kop[o] = k_operand(kt, kb0 + o % KBW, o / KBW);
    };
    auto read_vop = [&](int o, const unsigned char* vt) __attribute__((always_inline)) {
        vop[o] = v_operand(vt + VOFF, kb0 + o / (2 * (D / 32)), (o / (D / 32)) % 2, o % (D / 32));
    };
    // Per-lane LDS addresses of the operand reads for loops with constant
    // stage indices: K operand of K-step s at klb[s] + stage * TILE_B + (key
    // block) * 32 * RB; V operand of head-dimension block db at vlb[db] +
    // VOFF + stage * TILE_B + (key block * 32 + 16 u + 8 hf) * RB. The key
    // block and u, hf offsets keep the swizzles (they move whole rows within
    // a swizzle period).
    constexpr int NKL = D / 16, NVL = D / 32;
    constexpr int KOFF_MAX = (NST - 1) * TILE_B + (KBW - 1) * 32 * RB;
    constexpr int VOFF_MAX = (NST - 1) * TILE_B + ((KBW - 1) * 32 + 24) * RB;
    constexpr bool UNROLL = NST % 2 == 0 && KOFF_MAX < 65536 && VOFF_MAX < 65536;
    uint32_t klb[NKL], vlb[NVL];
    {
        const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)smem;
        const int krow = kb0 * 32 + n32;
#pragma unroll
        for (int s2 = 0; s2 < NKL; ++s2) klb[s2] = base + krow * RB + (((2 * s2 + hh) ^ swz_k<D>(krow)) << 4);
        const int vrow = kb0 * 32 + 4 * hh + e_tr;
#pragma unroll
        for (int db = 0; db < NVL; ++db) {
            const int lc = db * 4 + 2 * (grp & 1) + (q_tr >> 1);
            vlb[db] = base + VOFF + vrow * RB + ((lc ^ swz_v<D>(vrow)) << 4) + 8 * (q_tr & 1);
        }
    }
    typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
    auto read_kop_c = [&](int o, int stg) __attribute__((always_inline)) {
        const int kb = o % KBW, s2 = o / KBW;
        kop[o] = *(lds_cu32x4*)(uintptr_t)(klb[s2] + stg * TILE_B + kb * 32 * RB);
    };
    auto read_vop_c = [&](int o, int stg) __attribute__((always_inline)) {
        const int kb = o / (2 * (D / 32)), u = (o / (D / 32)) % 2, db = o % (D / 32);
        u32x2 part[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const uint32_t a = vlb[db] + stg * TILE_B + (kb * 32 + 16 * u + 8 * hf) * RB;
            const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
            part[hf] = __builtin_bit_cast(u32x2, r);
        }
        vop[o] = u32x4{part[0][0], part[0][1], part[1][0], part[1][1]};
    };
    // the V operands due in the first LA slots of the next iteration
    auto read_v_carry = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < LA && f < NPV; ++f)
            if (f % NQ == 0) read_vop(f / NQ, stage(tile));
    };

    // ---- running state -----------------------------------------------------
    // m_run: the reference max (log2 units, always finite); l_run: the sum of
    // the row's probabilities against it, the same in both lane halves. It is
    // register 0 of lacc, the accumulator of the row-sum products (registers
    // 1-3 are rows the selector leaves empty and stay 0).
    f32x16 oacc[NQ][D / 32];
    f32x4 lacc[NQ];
    float m_run[NQ], l_run[NQ], l_old[NQ];
    // Selector operand (A of the 16x16x32 row-sum product). Lane l holds A
    // row l % 16 over contraction slots 8*(l/16) .. +7; as B, a probability
    // block gives slot 8g + i of column c the probability of query c + 16*(g
    // odd) and key 8*(g >= 2) + i (g = l/16 of the supplying lane). Result
    // row 4g' of column c sits in register 0 of lane 16g' + c, whose query is
    // c + 16*(g' odd); that row must gather the slots of the groups g with
    // the same parity. So A row r is 1 on the slots of group g exactly when r
    // is 0 or 8 and g is even, or r is 4 or 12 and g is odd.
    u32x4 sel_ones;
    {
        const int r16 = lane & 15, g16 = lane >> 4;
        const bool on = (g16 & 1) ? (r16 == 4 || r16 == 12) : (r16 == 0 || r16 == 8);
        const uint32_t one2 = std::is_same<Tag, BF16>::value ? 0x3F803F80u : 0x3C003C00u;
        const uint32_t w1 = on ? one2 : 0u;
        sel_ones = u32x4{w1, w1, w1, w1};
    }
#pragma unroll
    for (int gq = 0; gq < NQ; ++gq) {
        m_run[gq] = 0.f;
        l_run[gq] = 0.f;
        l_old[gq] = 0.f;
        lacc[gq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[gq][db][r] = 0.f;
    }
    const float c = p.c;
    SAcc s_buf[2];   // scores of tile t (softmax) and t+1 (being multiplied)
    PAcc pq[2];      // probabilities of tile t (softmax) and t-1 (output product)

    // Product number i of K Q^T into S, order (s, kb, gq).
    auto qk_mfma = [&](int i, SAcc& S) __attribute__((always_inline)) {
        const int gq = i % NQ, kb = (i / NQ) % KBW, s = i / (NQ * KBW);
        const f32x16 zero = {};
        S[kb][gq] = mfma16<Tag>(kop[i / NQ], qop[gq][s], s == 0 ? zero : S[kb][gq]);
    };
    // Product number i of P V into O, order (kb, u, db, gq).
    auto pv_mfma = [&](int i, const PAcc& Pm) __attribute__((always_inline)) {
        const int gq = i % NQ, db = (i / NQ) % (D / 32), u = (i / (NQ * (D / 32))) % 2,
                  kb = i / (NQ * (D / 32) * 2);
        oacc[gq][db] = mfma16<Tag>(vop[i / NQ], Pm[gq][kb][u], oacc[gq][db]);
    };
    // Probability pair j of the lane: block (kb, gq) = ((j/8) % KBW, j / (8 KBW)),
    // result registers r, r+1 with r = 2 (j % 8); 16-key block u = r / 8.
    auto prob_pair = [&](int j, const SAcc& S, PAcc& Pm, float m) __attribute__((always_inline)) {
        const int gq = j / (8 * KBW), kb = (j / 8) % KBW, r = 2 * (j % 8);
        // masked scores are -inf and c > 0, so their probabilities are 0
        const float p0 = fast_exp2(fmaf(S[kb][gq][r], c, -m));
        const float p1 = fast_exp2(fmaf(S[kb][gq][r + 1], c, -m));
        Pm[gq][kb][r / 8][(r / 2) & 3] = pack2<Tag>(p0, p1);
    };
    // Row sums of 16-key block bj = (gq, kb, u) (pairs 4 bj .. 4 bj + 3) into
    // lacc: the sums use the rounded probabilities, as the output product does.
    auto row_sum_block = [&](int bj, const PAcc& Pm) __attribute__((always_inline)) {
        const int gq = bj / (2 * KBW), kb = (bj / 2) % KBW, u = bj % 2;
        lacc[gq] = mfma16x16<Tag>(sel_ones, Pm[gq][kb][u], lacc[gq]);
    };
    // Scores of `tile` past the rows' limits (causal, key length) -> -inf.
    auto mask_scores = [&](SAcc& S, int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
            const int qi = qw0 + gq * 32 + n32;
            const int lim = p.causal ? min(lim_hi, qi + 1) : lim_hi;
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (wkey0(tile) + kb * 32 + blk_row(r, hh) >= lim) S[kb][gq][r] = kNegInf;
        }
    };
    // Maximum of query block gq's scores in S over both lane halves (the
    // whole row of the tile), in log2 units; -inf when every key is masked.
    auto row_max = [&](int gq, const SAcc& S) __attribute__((always_inline)) -> float {
        float mq[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < KBW; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const int ch = (kb * 4 + r / 4) & 3;
                mq[ch] = fmaxf(mq[ch], fmaxf(S[kb][gq][r], S[kb][gq][r + 1]));
                mq[ch] = fmaxf(mq[ch], fmaxf(S[kb][gq][r + 2], S[kb][gq][r + 3]));
            }
        float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
        mx = fmaxf(mx, swap_halves(mx));
        return mx * c;  // -inf stays -inf (c > 0)
    };
    // Block gq after a sum left the range: move the reference to the exact
    // running max, rescale l (O by the caller, with the returned factor) and
    // redo the probabilities and their row sums. Both lane halves of a query
    // hold the same sums and decide alike.
    auto exact_max = [&](int gq, const SAcc& S, PAcc& Pm) __attribute__((always_inline)) -> float {
        const float mxs = row_max(gq, S);
        // nothing accumulated yet: the old reference carries no weight
        float m_new = l_old[gq] > 0.f ? fmaxf(m_run[gq], mxs) : mxs;
        if (m_new == kNegInf) m_new = m_run[gq];  // every key of the row masked so far
        const float alpha = l_old[gq] > 0.f ? fast_exp2(m_run[gq] - m_new) : 1.f;
        m_run[gq] = m_new;
#pragma unroll
        for (int j = 0; j < 8 * KBW; ++j) prob_pair(gq * 8 * KBW + j, S, Pm, m_new);
        lacc[gq] = f32x4{l_old[gq] * alpha, 0.f, 0.f, 0.f};
#pragma unroll
        for (int bj = gq * 2 * KBW; bj < (gq + 1) * 2 * KBW; ++bj) row_sum_block(bj, Pm);
        l_run[gq] = lacc[gq][0];
        return alpha;
    };
    // After the probabilities of a tile (and the products of the previous
    // one): blocks with a sum out of range take the exact-max path, and their
    // O is rescaled.
    auto fix_range = [&](const SAcc& S, PAcc& Pm) __attribute__((always_inline)) {
        // one test over all blocks first: every block's sum is then needed
        // before any branch, which keeps the probability work in place
        bool bad = false;
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) bad = bad || sum_out_of_range(l_run[gq]);
        if (__builtin_amdgcn_ballot_w64(bad) == 0) return;
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
            if (__builtin_amdgcn_ballot_w64(sum_out_of_range(l_run[gq])) == 0) continue;
            const float alpha = exact_max(gq, S, Pm);
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[gq][db][r] *= alpha;
        }
    };

    // ---- the key loop ---------------------------------------------------------
    // Iteration t (tile t's probabilities): wait for tile t+1, barrier, issue
    // the DMA of tile t+P into the stage of tile t-2 (its last reads completed
    // before the products of iteration t-1) -- with BAR2, at even t only, for
    // tiles t+1, t+2 and into the stages of t-3, t-2 --, read K(t+1); mask tile t's scores
    // where some row cannot see all its keys; then the products P(t-1) V(t-1)
    // and K(t+1) Q^T, one at a time, each followed by its share of tile t's
    // probability stages and row-sum products; check the sums; read V(t) for
    // the next iteration.
    // At t = 0 the output product multiplies zero probabilities; at the last
    // tile the score product reads a stale stage and its result is unused.
    auto iteration = [&](auto par, int t, auto stg) __attribute__((always_inline)) {
        constexpr int B = decltype(par)::value;
        constexpr int SG = decltype(stg)::value;  // stage of tile t when a constant (-1: from t)
        SAcc& s_cur = s_buf[B];
        SAcc& s_nxt = s_buf[B ^ 1];
        PAcc& p_cur = pq[B];
        PAcc& p_prv = pq[B ^ 1];
        if constexpr (BAR2) {
            // even t only: tiles t+1 and t+2 (read in iterations t and t+1)
            // have landed for every wave; after the barrier every wave is past
            // iteration t-1, so the stages of tiles t-3 and t-2 are free
            if constexpr (B == 0) {
                if (t + 1 < ntiles) wait_tile(min(t + 2, ntiles - 1), min(t + P - 1, ntiles - 1));
                barrier_nofence();
                // one wave-uniform guard for both loads (per call, the
                // compiler kept a copy of it in a VGPR, spilled, and reloaded
                // it after the barrier, a reload whose wait drained the DMA)
                if (wave < NIW) {
                    if (t + P < ntiles) issue_tile(t + P);
                    if (t + P + 1 < ntiles) issue_tile(t + P + 1);
                }
            }
        } else {
            if (t + 1 < ntiles) wait_tile(t + 1, min(t + P - 1, ntiles - 1));
            barrier_nofence();
            if (t + P < ntiles) issue_tile(t + P);
        }
        const unsigned char* kt = stage(t + 1);
        const unsigned char* vt = stage(t > 0 ? t - 1 : 0);
        constexpr int KSG = SG >= 0 ? (SG + 1) % NST : 0;        // stage of tile t+1
        constexpr int VSG = SG >= 0 ? (SG + NST - 1) % NST : 0;  // stage of tile t-1
        const int ksr = (t + 1) % NST, vsr = (t > 0 ? t - 1 : 0) % NST;
        if constexpr (SG >= 0) {
            // fresh names for the lane addresses each iteration, so that no
            // stage's sums of them are kept in registers across the loop
#pragma unroll
            for (int j = 0; j < NKL; ++j) asm volatile("" : "+v"(klb[j]));
#pragma unroll
            for (int j = 0; j < NVL; ++j) asm volatile("" : "+v"(vlb[j]));
        }
        if (wkey0(t) + KBW * 32 > wave_lim_min) mask_scores(s_cur, t);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) l_old[gq] = l_run[gq];
        // Slot k owns pairs [k NPAIR / NM, (k+1) NPAIR / NM); slot i runs the
        // exponentials of slot i's pairs, the scale-and-shift of slot i+1's,
        // the rounding of slot i-1's and the row sums of the blocks whose
        // last pair slot i-2 owns.
        float xs[NPAIR][2], es[NPAIR][2];
        auto pairs = [](int k) { return k * NPAIR / NM; };
        auto stage_shift = [&](int k) __attribute__((always_inline)) {
            if (k < 0 || k >= NM) return;
#pragma unroll
            for (int j = pairs(k); j < pairs(k + 1); ++j) {
                const int gq = j / (8 * KBW), kb = (j / 8) % KBW, r = 2 * (j % 8);
                // masked scores are -inf and c > 0, so their probabilities are 0
                xs[j][0] = fmaf(s_cur[kb][gq][r], c, -m_run[gq]);
                xs[j][1] = fmaf(s_cur[kb][gq][r + 1], c, -m_run[gq]);
            }
        };
        auto stage_exp = [&](int k) __attribute__((always_inline)) {
            if (k < 0 || k >= NM) return;
#pragma unroll
            for (int j = pairs(k); j < pairs(k + 1); ++j) {
                es[j][0] = fast_exp2(xs[j][0]);
                es[j][1] = fast_exp2(xs[j][1]);
            }
        };
        auto stage_round = [&](int k) __attribute__((always_inline)) {
            if (k < 0 || k >= NM) return;
#pragma unroll
            for (int j = pairs(k); j < pairs(k + 1); ++j) {
                const int gq = j / (8 * KBW), kb = (j / 8) % KBW, r = 2 * (j % 8);
                p_cur[gq][kb][r / 8][(r / 2) & 3] = pack2<Tag>(es[j][0], es[j][1]);
            }
        };
        auto stage_sum = [&](int k) __attribute__((always_inline)) {
            if (k < 0 || k >= NM) return;
#pragma unroll
            for (int j = pairs(k); j < pairs(k + 1); ++j)
                if (j % 4 == 3) row_sum_block(j / 4, p_cur);
        };
        stage_shift(0);
        // At head size 128 a wave in its product slots takes issue priority
        // over a wave of the same SIMD in its barrier, DMA or sum-check
        // phase (measured on gfx950: 1-2 % faster on every head-size-128
        // variant, long causal included; head size 64 unchanged, so it
        // keeps one priority).
        if constexpr (D == 128) __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            // operand reads for slot i + LA
            const int f = i + LA;
            if constexpr (SG >= 0) {
                // at t = 0 the output product multiplies zero probabilities:
                // any stage will do (stage 0 holds tile 0)
                if (f < NPV && f % NQ == 0) read_vop_c(f / NQ, VSG);
                if (f >= NPV && f < NM && (f - NPV) % NQ == 0) read_kop_c((f - NPV) / NQ, KSG);
                if (i < LA && i >= NPV && (i - NPV) % NQ == 0) read_kop_c((i - NPV) / NQ, KSG);
            } else if constexpr (UNROLL) {
                // the leftover tiles after the unrolled trips read through
                // the same lane bases with a run-time stage offset: no lane
                // index then stays live across the unrolled loop (it was
                // spilled there, and the spills cost HBM traffic)
                if (f < NPV && f % NQ == 0) read_vop_c(f / NQ, vsr);
                if (f >= NPV && f < NM && (f - NPV) % NQ == 0) read_kop_c((f - NPV) / NQ, ksr);
                if (i < LA && i >= NPV && (i - NPV) % NQ == 0) read_kop_c((i - NPV) / NQ, ksr);
            } else {
                if (f < NPV && f % NQ == 0) read_vop(f / NQ, vt);
                if (f >= NPV && f < NM && (f - NPV) % NQ == 0) read_kop((f - NPV) / NQ, kt);
                if (i < LA && i >= NPV && (i - NPV) % NQ == 0) read_kop((i - NPV) / NQ, kt);
            }
            if (i < NPV) pv_mfma(i, p_prv); else qk_mfma(i - NPV, s_nxt);
            stage_exp(i);
            stage_shift(i + 1);
            stage_round(i - 1);
            stage_sum(i - 2);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (D == 128) __builtin_amdgcn_s_setprio(0);
        stage_round(NM - 1);
        stage_sum(NM - 2);
        stage_sum(NM - 1);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) l_run[gq] = lacc[gq][0];
        fix_range(s_cur, p_cur);
        if constexpr (SG >= 0 || UNROLL) {
#pragma unroll
            for (int f = 0; f < LA && f < NPV; ++f)
                if (f % NQ == 0) read_vop_c(f / NQ, SG >= 0 ? SG : t % NST);
        } else {
            read_v_carry(t);
        }
    };

    // The Q operands and tile 0 load together (one wait covers both); the
    // Q loads go first, as they do not wait for the key length. The rest of
    // the ring goes out after the wait.
    if constexpr (UNROLL) {
        // the unrolled loop's first output product reads the V stage of
        // "tile -1" (stage NST - 1) against zero probabilities: clear it so
        // that no stale bits meet the zeros (the barrier before the first
        // iteration orders these writes)
        u32x4* vz = reinterpret_cast<u32x4*>(smem + VOFF + (NST - 1) * TILE_B);
        for (int i = tid; i < TILE_B / 16; i += 256 * KSPLIT) vz[i] = u32x4{0u, 0u, 0u, 0u};
    }
    if (ntiles > 0) issue_tile(0);
    wait_vmcnt<0>();
    for (int t = 1; t < min(P, ntiles); ++t) issue_tile(t);
    if constexpr (QLDS) {
        barrier_nofence();  // the staged Q rows have landed for every wave
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const int row = wq * 32 * NQ + gq * 32 + n32;
                qop[gq][s] = *reinterpret_cast<const u32x4*>(smem + QOFF + row * RB +
                                                             (((2 * s + hh) ^ swz_k<D>(row)) << 4));
            }
    }
    if (ntiles > 0) {
        if constexpr (!QLDS) barrier_nofence();
#pragma unroll
        for (int o = 0; o < NK; ++o) read_kop(o, stage(0));
#pragma unroll
        for (int i = 0; i < NQK; ++i) qk_mfma(i, s_buf[0]);
        read_v_carry(0);
        // The reference of each row starts at its exact maximum over this
        // wave's first tile. Masks only grow with the key index, so a row
        // with no valid key in that tile has none in the wave's later tiles
        // either; its reference stays 0 and its sum 0.
        if (wkey0(0) + KBW * 32 > wave_lim_min) mask_scores(s_buf[0], 0);
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq) {
            const float mx = row_max(gq, s_buf[0]);
            m_run[gq] = mx == kNegInf ? 0.f : mx;
        }
#pragma unroll
        for (int gq = 0; gq < NQ; ++gq)
#pragma unroll
            for (int kb = 0; kb < KBW; ++kb) pq[1][gq][kb][0] = pq[1][gq][kb][1] = u32x4{0u, 0u, 0u, 0u};
    }
    // register set 0 serves the even tiles (the BAR2 barrier relies on it)
    int t = 0;
    // Rings whose K (and V) tiles fit the 64 KiB reach of the ds_read
    // immediate offset run NST tiles per trip with each stage index a
    // constant: every operand address is then a per-lane base plus an
    // immediate, and the loop issues no address additions (measured on
    // gfx950: 1-8 % faster on those variants, 2-4 % on the three-per-SIMD
    // one once the DMA addressing no longer held per-lane 64-bit pointers).
    if constexpr (UNROLL) {
        for (; t + NST <= ntiles; t += NST) {
            for_each_stage(
                [&](auto kc) __attribute__((always_inline)) {
                    constexpr int K = decltype(kc)::value;
                    iteration(int_c<K & 1>{}, t + K, int_c<K>{});
                },
                std::make_integer_sequence<int, NST>{});
        }
    }
    for (; t + 1 < ntiles; t += 2) {
        iteration(int_c<0>{}, t, int_c<-1>{});
        iteration(int_c<1>{}, t + 1, int_c<-1>{});
    }
    if (t < ntiles) iteration(int_c<0>{}, t, int_c<-1>{});
    if (ntiles > 0) {
        // products of the last tile (its first V operands came with the carry)
#pragma unroll
        for (int o = 0; o < NV; ++o) {
            if (o * NQ < LA) continue;
            if constexpr (UNROLL) read_vop_c(o, (ntiles - 1) % NST);
            else read_vop(o, stage(ntiles - 1));
        }
        if ((ntiles - 1) & 1) {
#pragma unroll
            for (int i = 0; i < NPV; ++i) pv_mfma(i, pq[1]);
        } else {
#pragma unroll
            for (int i = 0; i < NPV; ++i) pv_mfma(i, pq[0]);
        }
    }
    __syncthreads();  // all DMA landed (last wait was vmcnt(0)) and all reads done

    // ---- merge the two key halves (KSPLIT = 2) ------------------------------
    // Lane (n32, h) of waves w and w+4 holds the same queries and the same
    // rows of O^T over disjoint keys: O = O_a 2^(m_a - m) + O_b 2^(m_b - m),
    // where a half with nothing accumulated (l = 0) has no weight. Each half
    // finishes half of the head dimension: half kh keeps the 32-column blocks
    // [kh DB/2, (kh+1) DB/2) and hands the others, with its (m, l), to its
    // partner through LDS. Both halves then compute the same (m, l).
    constexpr int DB = D / 32;
    constexpr int DBH = KSPLIT == 2 ? DB / 2 : DB;  // blocks finished by each wave
    // The rest runs with the wave's key half as a constant, so that the
    // accumulator blocks it finishes are indexed at compile time.
    auto finish = [&](auto khc) __attribute__((always_inline)) {
        constexpr int KH = decltype(khc)::value;
        constexpr int db0 = KSPLIT == 2 ? KH * DBH : 0;  // first block this wave finishes
        if constexpr (KSPLIT == 2) {
            float* mine = reinterpret_cast<float*>(smem) + (KH * 4 + wq) * (MRG_W / 4);
            const float* theirs = reinterpret_cast<const float*>(smem) + ((KH ^ 1) * 4 + wq) * (MRG_W / 4);
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
#pragma unroll
                for (int j = 0; j < DBH; ++j) {
                    const int db = (KH ^ 1) * DBH + j;  // the partner's blocks
#pragma unroll
                    for (int r = 0; r < 16; ++r) mine[((gq * DBH + j) * 16 + r) * 64 + lane] = oacc[gq][db][r];
                }
                mine[(NQ * DBH * 16 + 2 * gq) * 64 + lane] = m_run[gq];
                mine[(NQ * DBH * 16 + 2 * gq + 1) * 64 + lane] = l_run[gq];
            }
            __syncthreads();
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
                const float mb = theirs[(NQ * DBH * 16 + 2 * gq) * 64 + lane];
                const float lb = theirs[(NQ * DBH * 16 + 2 * gq + 1) * 64 + lane];
                // l holds whole-row sums: both lane halves of a query decide alike
                const float la = l_run[gq];
                const float ma = m_run[gq];
                const float mm = la == 0.f ? mb : (lb == 0.f ? ma : fmaxf(ma, mb));
                const float wa = la == 0.f ? 0.f : fast_exp2(ma - mm);
                const float wb = lb == 0.f ? 0.f : fast_exp2(mb - mm);
                // the same expression in both halves (KH 0 holds "a"): identical bits
                const float l0 = KH == 0 ? la : lb, w0 = KH == 0 ? wa : wb;
                const float l1 = KH == 0 ? lb : la, w1 = KH == 0 ? wb : wa;
                m_run[gq] = mm;
                l_run[gq] = l0 * w0 + l1 * w1;
#pragma unroll
                for (int j = 0; j < DBH; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        oacc[gq][db0 + j][r] = oacc[gq][db0 + j][r] * wa + theirs[((gq * DBH + j) * 16 + r) * 64 + lane] * wb;
            }
            __syncthreads();
        }

        // ---- epilogue of a key range: the rows' records --------------------------
        // Lane (n32, h) holds o[d] for d = db*32 + 8jj + 4h + e, e = 0..3: one
        // 16-byte store each.
        if constexpr (SPLIT) {
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
                const int qi = qw0 + gq * 32 + n32;
                if (qi >= p.Sq) continue;
                const float lt = l_run[gq];
                float* rec = p.ws + ((((int64_t)b * p.H + h) * p.Sq + qi) * p.n_split + split) * (D + 4);
                if (hh == 0 && KH == 0) {
                    rec[0] = lt > 0.f ? m_run[gq] : kNegInf;
                    rec[1] = lt;
                }
#pragma unroll
                for (int j = 0; j < DBH; ++j)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int db = db0 + j;
                        const f32x16& ov = oacc[gq][db];
                        *reinterpret_cast<f32x4*>(rec + 4 + db * 32 + 8 * jj + 4 * hh) =
                            f32x4{ov[4 * jj], ov[4 * jj + 1], ov[4 * jj + 2], ov[4 * jj + 3]};
                    }
            }
            return;
        }

        // ---- epilogue: O = O_acc / l, LSE = (m + log2 l) ln 2 -------------------
        // Each wave stages its blocks of the head dimension; the rows of a query
        // group are then stored by both of its waves, half each. An 8-byte
        // write pass covers 16 consecutive rows on 32 banks, where rows OROW
        // elements apart meet in pairs (r and r + 8): rows with bit 3 set swap
        // the two 8-byte halves of each 16-byte chunk, and the store loop
        // swaps them back.
        {
            T* Os = reinterpret_cast<T*>(smem) + wq * 32 * NQ * OROW;
#pragma unroll
            for (int gq = 0; gq < NQ; ++gq) {
                const float lt = l_run[gq];
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                const int qi = qw0 + gq * 32 + n32;
                if (hh == 0 && KH == 0 && p.lse != nullptr && qi < p.Sq)
                    p.lse[((int64_t)b * p.H + h) * p.Sq + qi] = lt > 0.f ? (m_run[gq] + log2f(lt)) * kLn2 : kNegInf;
                T* orow = Os + (gq * 32 + n32) * OROW;
                const int half = hh ^ ((n32 >> 3) & 1);
#pragma unroll
                for (int j = 0; j < DBH; ++j)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int db = db0 + j;
                        const int d0 = db * 32 + 8 * jj + 4 * half;
                        const f32x16& ov = oacc[gq][db];
                        const u32x2 pk2 = {pack2<Tag>(ov[4 * jj] * inv, ov[4 * jj + 1] * inv),
                                           pack2<Tag>(ov[4 * jj + 2] * inv, ov[4 * jj + 3] * inv)};
                        *reinterpret_cast<u32x2*>(orow + d0) = pk2;
                    }
            }
        }
        __syncthreads();
        {
            const T* Os = reinterpret_cast<const T*>(smem) + wq * 32 * NQ * OROW;
            for (int cidx = KH * 64 + lane; cidx < 32 * NQ * CPR; cidx += 64 * KSPLIT) {
                const int row = cidx / CPR, cc = cidx - row * CPR;
                const int qi = qw0 + row;
                if (qi < p.Sq) {
                    u32x4 val = *reinterpret_cast<const u32x4*>(Os + row * OROW + cc * 8);
                    if ((row >> 3) & 1) val = u32x4{val[2], val[3], val[0], val[1]};
                    // streaming stores: O is written once and not read here
                    // (measured on gfx950: 1-3.5 % faster, most on short key walks)
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(op + (int64_t)qi * p.sq.s + cc * 8));
                }
            }
        }
    };
    if constexpr (KSPLIT == 1) {
        finish(int_c<0>{});
    } else {
        if (kh == 0) finish(int_c<0>{}); else finish(int_c<1>{});
    }
}

// Causal tiles of all the heads of an XCD interleaved (longest first) while
// those heads' K and V take at most this many bytes: measured on gfx950, the
// interleave cut 11-24 % at 4-8 MiB (B4 H16 S2048, B8 H16 S1024, B2 H32 S4096,
// head size 64) and gained nothing at 16 MiB (B2 H16 S8192, head size 128),
// where the competing heads' K/V no longer fit the XCD's 4 MiB L2 and the
// HBM reads grew 1.75x.
constexpr int64_t kCausalMixBytes = int64_t(8) << 20;

template <typename Tag, int D, int NQ, int BN, int NST, int KSPLIT, int OCC, bool SPLIT>
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
    // c > 0 keeps masked scores (-inf) at probability 0; scale 0 becomes the
    // limit scale -> 0+, the same uniform attention
    p.c = a.scale > 0.f ? a.scale * kLog2e : 1e-30f;
    p.causal = a.causal ? 1 : 0;
    p.n_qtiles = (a.Sq + BM - 1) / BM;
    p.ws = static_cast<float*>(a.ws);
    p.n_split = SPLIT ? a.n_split : 1;
    // key ranges of whole 64-key blocks (whole tiles of every variant)
    static_assert(64 % BN == 0, "key ranges must be whole tiles");
    p.chunk = SPLIT ? (a.Sk + a.n_split * 64 - 1) / (a.n_split * 64) * 64 : a.Sk;
    const int64_t grid = (int64_t)p.n_qtiles * a.B * a.H * p.n_split;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    const int64_t bh = (int64_t)a.B * a.H;
    const int64_t xcd_kv_bytes = bh / 8 * (int64_t)a.Sk * D * 2 * 2;
    p.causal_heads = (a.causal && !SPLIT && bh % 8 == 0 && xcd_kv_bytes <= kCausalMixBytes) ? (int)(bh / 8) : 0;
    hipLaunchKernelGGL((fwd_prefill16_kernel<Tag, D, NQ, BN, NST, KSPLIT, OCC, SPLIT>), dim3((unsigned)grid),
                       dim3(256 * KSPLIT), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !SPLIT) return e;
    return run_splitk_merge(a, a.n_split, a.ws, stream);
}

// ---- tile variants and their choice ----------------------------------------
// Tile sizes are not probed at run time: the candidates below are compiled in
// (none uses scratch memory at its waves per SIMD), and
// a table made offline by timing every candidate over a grid of shapes
// (tile_table.inc) names the variant per head size, masking, key length and
// query rows.
struct Variant16 {
    int nq, bn, nst, ksplit, lds;
    hipError_t (*run[2][2])(const FwdArgs&, hipStream_t);  // [whole keys, key splits][fp16, bf16]
};
#define ATTN_VARIANT16(D, NQ, BN, NST, KS, OCC)                                                        \
    {NQ, BN, NST, KS, lds_bytes16(D, NQ, BN, NST, KS),                                                  \
     {{&launch16<F16, D, NQ, BN, NST, KS, OCC, false>, &launch16<BF16, D, NQ, BN, NST, KS, OCC, false>}, \
      {&launch16<F16, D, NQ, BN, NST, KS, OCC, true>, &launch16<BF16, D, NQ, BN, NST, KS, OCC, true>}}}
const Variant16 kVariants64[] = {
    ATTN_VARIANT16(64, 1, 64, 5, 1, 2),  // 0: 128 queries x 64 keys, 4 waves
    ATTN_VARIANT16(64, 1, 64, 4, 1, 2),  // 1: same, shorter ring
    ATTN_VARIANT16(64, 2, 64, 6, 2, 2),  // 2: 256 queries, 8 waves in two key halves
    ATTN_VARIANT16(64, 1, 64, 6, 2, 2),  // 3: 128 queries, 8 waves in two key halves
    ATTN_VARIANT16(64, 1, 32, 4, 1, 3),  // 4: 128 queries x 32 keys, 4 waves, three per SIMD
    ATTN_VARIANT16(64, 2, 32, 6, 1, 2),  // 5: 256 queries x 32 keys, 4 waves, two per SIMD
};
const Variant16 kVariants128[] = {
    ATTN_VARIANT16(128, 1, 32, 5, 1, 2),  // 0: 128 queries x 32 keys, 4 waves
    ATTN_VARIANT16(128, 1, 32, 4, 1, 2),  // 1: same, shorter ring
    ATTN_VARIANT16(128, 1, 64, 4, 2, 2),  // 2: 128 queries x 64 keys, 8 waves in two key halves
    ATTN_VARIANT16(128, 1, 64, 5, 2, 2),  // 3: same, deeper ring (all 160 KiB of LDS)
};
#undef ATTN_VARIANT16
constexpr int kNumVariants64 = sizeof(kVariants64) / sizeof(kVariants64[0]);
constexpr int kNumVariants128 = sizeof(kVariants128) / sizeof(kVariants128[0]);

#include "tile_table.inc"

// With key ranges the grid holds about two workgroups per compute unit: the
// 4-wave, 128-query variant with the 4-stage ring was the fastest on every
// few-head shape measured on gfx950 (32 to 128 query tiles over 4096 to
// 32768 keys, both head sizes), ahead of the 8-wave ones at half the ranges.
constexpr int kRangeTile64 = 1;
constexpr int kRangeTile128 = 1;
static_assert(kRangeTile64 < kNumVariants64 && kRangeTile128 < kNumVariants128, "key-range variant");

// Bucket of x on a log2 grid starting at 2^lo with n points (nearest point).
int log2_bucket(int64_t x, int lo, int n) {
    int e = 0;
    while (e < 62 && (int64_t(1) << (e + 1)) <= x) ++e;  // floor(log2 x)
    // round: x >= 2^e * sqrt(2) goes up
    if (e < 62 && (double)x >= (double)(int64_t(1) << e) * 1.4142135623730951) ++e;
    const int i = e - lo;
    return i < 0 ? 0 : (i >= n ? n - 1 : i);
}

}  // namespace

int prefill16_tile_count(int d) { return d == 64 ? kNumVariants64 : d == 128 ? kNumVariants128 : 0; }

bool prefill16_tile_info(int d, int tile, TileInfo* out) {
    if (tile < 0 || tile >= prefill16_tile_count(d)) return false;
    const Variant16& v = d == 64 ? kVariants64[tile] : kVariants128[tile];
    out->rows = 4 * 32 * v.nq;
    out->keys = v.bn;
    out->waves = 4 * v.ksplit;
    out->stages = v.nst;
    out->lds_bytes = v.lds;
    return true;
}

int prefill16_tile_choice(int B, int H, int Sq, int Sk, int d, int causal, int n_split) {
    if (n_split > 1) return d == 128 ? kRangeTile128 : kRangeTile64;
    const int r = log2_bucket((int64_t)B * H * Sq, kTuneRowsLog2Min, kTuneRowsBuckets);
    const int k = log2_bucket(Sk, kTuneKeysLog2Min, kTuneKeysBuckets);
    return kTileTable[d == 128 ? 1 : 0][causal ? 1 : 0][r][k];
}

hipError_t run_prefill16(const FwdArgs& a, hipStream_t stream) {
    const int tile = a.tile >= 0 ? a.tile : prefill16_tile_choice(a.B, a.H, a.Sq, a.Sk, a.d, a.causal, a.n_split);
    if (tile < 0 || tile >= prefill16_tile_count(a.d)) return hipErrorInvalidValue;
    const Variant16& v = a.d == 128 ? kVariants128[tile] : kVariants64[tile];
    if (a.n_split > 1 && a.ws == nullptr) return hipErrorInvalidValue;
    return v.run[a.n_split > 1 ? 1 : 0][a.dtype == 2 ? 1 : 0](a, stream);
}

}  // namespace attn
