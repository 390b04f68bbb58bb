// Fused QKV projection for bf16 / fp16: one matrix product of the tokens
// with the concatenated weight, written straight into Q, K and V.
//
// Method (chapter "2. 自注意力机制算子…以及FlashAttention优化", §2.1): the
// projections X W_Q, X W_K and X W_V are done as one product with the three
// weights side by side ([D, 3 Hd]) and then split. Here the split is part of
// the store: output column n = t*Hd + h*d + c goes to tensor t (Q, K, V),
// head h, dimension c, in the layout the attention kernel reads ([B,H,S,d],
// [B,S,H,d] or the head-group split, page "WebGPU 算子优化…", section "QKV
// 矩阵的内存合并模式选择").
//
// Y = X W^T with X [M = B*S, K = D] and the weight stored out-major,
// w[n][i] (as a linear layer keeps it), so both operands of the matrix
// product are contiguous along the contraction.
//
// Mapping to gfx950:
//   * Two tilings. Tiling 0: 192 x 128 output tile per workgroup (192 weight
//     rows = output columns, 128 token rows), 4 waves of 96 x 64 (3 x 2
//     blocks of 32 x 32), two workgroups per CU. Tiling 1: 256 x 256, 8
//     waves of 128 x 64 (4 x 2 blocks), one workgroup per CU; it loads a
//     third fewer bytes per product but has half as many workgroups, so it
//     is taken only when it needs clearly fewer rounds of workgroups over
//     the CUs than tiling 0 (large products).
//   * The products are computed transposed, Y^T = W X^T, on 32x32x16
//     matrix-core blocks: A = weight rows, B = token rows. Each K-step of 16
//     reads 5 (6) operands from LDS for 6 (8) products, which keeps LDS
//     reads below what the LDS delivers at full matrix-core rate.
//   * K steps of 64: the X and W tiles go global -> LDS by direct DMA loads
//     into a two-stage ring (one tile ahead), rows of 128 B with their
//     16-byte chunks XOR-swizzled so the ds_read_b128 operand reads are free
//     of bank conflicts. A stage is 40 KiB (64 KiB).
//   * Operands are read one 16-deep step ahead, one read after each
//     product; the barrier of a tile sits after the first product of its
//     last step, so the queued product covers it.
//   * When the grid is a multiple of 8, consecutive tiles (token-row major)
//     go to one XCD, so its L2 serves their shared X and W reads.
//   * Epilogue: fp32 accumulators -> storage type (round to nearest even)
//     -> LDS -> 16-byte non-temporal stores, each chunk of 8 columns placed
//     by (t, h, c).
//   * Rows past M and columns past N reread the last valid row (finite) and
//     are not stored.
#include "device_common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int QBK = 64;         // contraction per stage
constexpr int QROW = QBK * 2;   // bytes per LDS row
constexpr int QNST = 2;

typedef __attribute__((address_space(3))) void lds_void_q;

struct QkvParams {
    const void* x;
    const void* w;
    void* out[3];
    int M, N, K;   // B*S, 3*H*d, D
    int S, H, d;
    Strides so;    // output layout
    int n_ntiles;  // column tiles
    int remap;     // grid size is a multiple of 8: contiguous tile ranges per XCD
};

template <int N> __device__ __forceinline__ void qwait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Direct global -> LDS load of 16 bytes per lane (see the attention kernel).
__device__ __forceinline__ void qdma16(const void* src, uint32_t lds_addr) {
    asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ void qbarrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row.
__device__ __forceinline__ int qswz(int row) { return (row >> 1) & 7; }

// A tiling: BM token rows x BN output columns per workgroup, NW waves on a
// WGM x (NW / WGM) grid, WPC workgroups per CU.
template <int BM_, int BN_, int NW_, int WGM_, int WPC_>
struct QTiling {
    static constexpr int BM = BM_, BN = BN_, NW = NW_, WGM = WGM_, WPC = WPC_;
    static constexpr int NT = NW * 64;
    static constexpr int WGN = NW / WGM;
    static constexpr int QWM = BM / WGM / 32;   // 32-row blocks per wave
    static constexpr int QWN = BN / WGN / 32;   // 32-column blocks per wave
    static constexpr int XTILE = BM * QROW;     // bytes of the X tile
    static constexpr int WTILE = BN * QROW;     // bytes of the W tile
    static constexpr int STAGE = XTILE + WTILE; // X tile, then W tile
    static constexpr int OROW = BN + 8;         // output staging row (elements)
    static constexpr int RING = QNST * STAGE, OUT = BM * OROW * 2;
    static constexpr int LDS = RING > OUT ? RING : OUT;
    static_assert(QWM * WGM * 32 == BM && QWN * WGN * 32 == BN, "waves cover the tile");
    static_assert(LDS <= 160 * 1024, "LDS of one workgroup");
};
using QTiling0 = QTiling<128, 192, 4, 2, 2>;
using QTiling1 = QTiling<256, 256, 8, 4, 1>;

template <typename Tag, typename C>
__global__ __launch_bounds__(C::NT, C::WPC) void qkv_proj_kernel(QkvParams p) {
    constexpr int QNT = C::NT, QWM = C::QWM, QWN = C::QWN, QXTILE = C::XTILE, QWTILE = C::WTILE;
    constexpr int QSTAGE = C::STAGE, QOROW = C::OROW, QBM = C::BM, QBN = C::BN;
    using T = uint16_t;
    __shared__ __align__(16) unsigned char smem[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WGN;  // block of token rows of this wave
    const int wn = wave % C::WGN;  // block of output columns of this wave
    const int n32 = lane & 31;
    const int hh = lane >> 5;

    const int G = gridDim.x;
    const int g = blockIdx.x;
    const int wg = p.remap ? (g & 7) * (G >> 3) + (g >> 3) : g;
    const int tm = wg / p.n_ntiles;
    const int tn = wg - tm * p.n_ntiles;
    const int m0 = tm * QBM, n0 = tn * QBN;

    const T* xp = static_cast<const T*>(p.x);
    const T* wp = static_cast<const T*>(p.w);

    // DMA slots: thread-slot i*QNT + tid of a tile is chunk (row, pc) and
    // holds logical chunk pc ^ swz(row) of that row (rows clamped to valid).
    constexpr int DMAX = QXTILE / 16 / QNT;  // loads per thread for X
    constexpr int DMAW = QWTILE / 16 / QNT;  // loads per thread for W
    static_assert(DMAX * 16 * QNT == QXTILE && DMAW * 16 * QNT == QWTILE, "tiles split over lanes");
    int64_t xoff[DMAX], woff[DMAW];
#pragma unroll
    for (int i = 0; i < DMAX; ++i) {
        const int slot = i * QNT + tid;
        const int row = slot / 8, pc = slot % 8;
        xoff[i] = (int64_t)min(m0 + row, p.M - 1) * p.K + (pc ^ qswz(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < DMAW; ++i) {
        const int slot = i * QNT + tid;
        const int row = slot / 8, pc = slot % 8;
        woff[i] = (int64_t)min(n0 + row, p.N - 1) * p.K + (pc ^ qswz(row)) * 8;
    }
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void_q*)smem;
    auto issue = [&](int kt) __attribute__((always_inline)) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds_base + (kt % QNST) * QSTAGE + wave * 1024);
        const int64_t k0 = (int64_t)kt * QBK;
#pragma unroll
        for (int i = 0; i < DMAX; ++i) qdma16(xp + xoff[i] + k0, st + i * QNT * 16);
#pragma unroll
        for (int i = 0; i < DMAW; ++i) qdma16(wp + woff[i] + k0, st + QXTILE + i * QNT * 16);
    };
    // operand of a 32-row block (rows rb*32.., K-step s) from a tile of 128-B rows
    auto operand = [&](const unsigned char* tile, int rb, int s) __attribute__((always_inline)) -> u32x4 {
        const int row = rb * 32 + n32;
        const int lc = 2 * s + hh;
        return *reinterpret_cast<const u32x4*>(tile + row * QROW + ((lc ^ qswz(row)) << 4));
    };

    f32x16 acc[QWN][QWM];  // [n block][m block] of Y^T
#pragma unroll
    for (int a = 0; a < QWN; ++a)
#pragma unroll
        for (int b2 = 0; b2 < QWM; ++b2)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b2][r] = 0.f;

    // Operand o of a K-step: o < QWN is W block wn*QWN + o, else X block
    // wm*QWM + o - QWN. They are double-buffered in registers: while the
    // products of K-step s run, the operands of K-step s+1 are read, one
    // after each product.
    constexpr int NO = QWN + QWM;  // operands per K-step
    constexpr int NP = QWN * QWM;  // products per K-step
    static_assert(NO < NP, "each operand read follows a product");
    auto read_op = [&](const unsigned char* st, int s, int o) __attribute__((always_inline)) -> u32x4 {
        return o < QWN ? operand(st + QXTILE, wn * QWN + o, s) : operand(st, wm * QWM + (o - QWN), s);
    };
    u32x4 op[2][NO];
    const int nk = p.K / QBK;
    issue(0);
    qwait_vmcnt<0>();
    qbarrier();
    if (nk > 1) issue(1);
#pragma unroll
    for (int o = 0; o < NO; ++o) op[0][o] = read_op(smem, 0, o);
    for (int kt = 0; kt < nk; ++kt) {
        const unsigned char* cur = smem + (kt % QNST) * QSTAGE;
        const unsigned char* nxt = smem + ((kt + 1) % QNST) * QSTAGE;
        const bool more = kt + 1 < nk;
#pragma unroll
        for (int s = 0; s < QBK / 16; ++s) {
            const u32x4* use = op[s & 1];
            u32x4* fill = op[(s & 1) ^ 1];
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int a = j / QWM, b2 = j % QWM;
                acc[a][b2] = mfma16<Tag>(use[a], use[QWN + b2], acc[a][b2]);
                if (s + 1 < QBK / 16) {
                    if (j < NO) fill[j] = read_op(cur, s + 1, j);
                } else if (more) {
                    // Last K-step of tile kt, after its first product (the
                    // operands of this K-step are already in registers):
                    // tile kt+1 has landed (this thread's loads) and, after
                    // the barrier, every wave is done reading tile kt, whose
                    // stage then takes tile kt+2. The operands of tile
                    // kt+1's first K-step follow the remaining products.
                    if (j == 0) {
                        qwait_vmcnt<0>();
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): own reads of tile kt done
                        qbarrier();
                        if (kt + 2 < nk) issue(kt + 2);
                    }
                    if (j >= 1 && j - 1 < NO) fill[j - 1] = read_op(nxt, 0, j - 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __syncthreads();  // all DMA landed and all operand reads done

    // ---- epilogue: Y tile (rows m, columns n) in LDS, then 16-byte stores ---
    // acc[a][b2] register r of lane (n32, hh): column n = (wn*QWN+a)*32 +
    // blk_row(r, hh) of the tile, row m = (wm*QWM+b2)*32 + n32.
    // An 8-byte write pass covers 16 lanes (16 consecutive rows) on 32
    // banks; rows QOROW elements apart meet in pairs, rows r and r + 8. Rows
    // with bit 3 set swap the two 8-byte halves of each 16-byte chunk, which
    // moves them onto the free banks (measured on gfx950: bank conflict
    // cycles down by two thirds); the store loop swaps them back.
    T* Ys = reinterpret_cast<T*>(smem);
#pragma unroll
    for (int a = 0; a < QWN; ++a)
#pragma unroll
        for (int b2 = 0; b2 < QWM; ++b2) {
            const int row = (wm * QWM + b2) * 32 + n32;
            const int half = hh ^ ((row >> 3) & 1);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int col = (wn * QWN + a) * 32 + 8 * g4 + 4 * half;
                const f32x16& v = acc[a][b2];
                const u32x2 pk = {pack2<Tag>(v[4 * g4], v[4 * g4 + 1]), pack2<Tag>(v[4 * g4 + 2], v[4 * g4 + 3])};
                *reinterpret_cast<u32x2*>(Ys + row * QOROW + col) = pk;
            }
        }
    __syncthreads();
    // Each thread keeps one 16-byte column chunk of the tile and walks rows
    // RPS apart: the chunk's tensor, head and column are divided out once,
    // and the (batch, token) of its rows advance by addition.
    constexpr int CPW = QBN / 8;    // 16-byte chunks per tile row
    constexpr int RPS = QNT / CPW;  // rows per sweep of the workgroup
    const int HD = p.H * p.d;
    const int cc = tid % CPW, n = n0 + cc * 8;
    if (tid < RPS * CPW && n < p.N) {
        const int t = n / HD, j = n - t * HD;
        const int h = j / p.d, c = j - h * p.d;
        T* const obase = static_cast<T*>(p.out[t]) + p.so.head(0, h) + c;
        int row = tid / CPW;
        int m = m0 + row;
        int b = m / p.S, s = m - b * p.S;
        for (; row < QBM && m < p.M; row += RPS, m += RPS) {
            u32x4 val = *reinterpret_cast<const u32x4*>(Ys + row * QOROW + cc * 8);
            if ((row >> 3) & 1) val = u32x4{val[2], val[3], val[0], val[1]};
            // streaming stores: the outputs of all workgroups leave at the end
            // of the launch at once, which non-temporal stores drain faster
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(obase + b * p.so.b + (int64_t)s * p.so.s));
            s += RPS;
            while (s >= p.S) {
                s -= p.S;
                ++b;
            }
        }
    }
}

template <typename C>
int64_t qkv_tiles(int M, int N) {
    return (int64_t)((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
}

template <typename C>
hipError_t launch_qkv(const QkvArgs& a, QkvParams p, hipStream_t stream) {
    p.n_ntiles = (p.N + C::BN - 1) / C::BN;
    const int64_t grid = qkv_tiles<C>(p.M, p.N);
    if (grid > 0x7fffffff || grid == 0) return grid == 0 ? hipSuccess : hipErrorInvalidValue;
    p.remap = (grid % 8 == 0) ? 1 : 0;
    if (a.dtype == 2)
        hipLaunchKernelGGL((qkv_proj_kernel<BF16, C>), dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
    else
        hipLaunchKernelGGL((qkv_proj_kernel<F16, C>), dim3((unsigned)grid), dim3(C::NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int qkv_proj_tiling(int M, int N, int n_cu) {
    // Rounds of workgroups over the CUs for each tiling; tiling 1 costs about
    // 1.1 rounds of tiling 0 per round (measured on gfx950: 375 against 457 us
    // for M 16384, N 6144, D 2048, where it needs 6 rounds against 8).
    const int64_t cu = n_cu > 0 ? n_cu : 256;
    const int64_t r0 = (qkv_tiles<QTiling0>(M, N) + QTiling0::WPC * cu - 1) / (QTiling0::WPC * cu);
    const int64_t r1 = (qkv_tiles<QTiling1>(M, N) + QTiling1::WPC * cu - 1) / (QTiling1::WPC * cu);
    return 11 * r1 < 10 * r0 ? 1 : 0;
}

hipError_t run_qkv_proj(const QkvArgs& a, hipStream_t stream) {
    QkvParams p;
    p.x = a.x;
    p.w = a.w;
    p.out[0] = a.q;
    p.out[1] = a.k;
    p.out[2] = a.v;
    p.M = a.B * a.S;
    p.N = 3 * a.H * a.d;
    p.K = a.D;
    p.S = a.S;
    p.H = a.H;
    p.d = a.d;
    p.so = make_strides(a.layout, a.H, a.S, a.d);
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        n_cu = 0;
    return qkv_proj_tiling(p.M, p.N, n_cu) == 1 ? launch_qkv<QTiling1>(a, p, stream)
                                               : launch_qkv<QTiling0>(a, p, stream);
}

}  // namespace attn
