/*
 * libattn: fused scaled-dot-product attention forward for MI355X (gfx950).
 *
 * Computes, for every batch b, head h and query row i,
 *     S_ij = scale * q_i . k_j                 (scores)
 *     P_ij = exp(S_ij - m_i) / l_i             (softmax along the keys)
 *     O_i  = sum_j P_ij v_j                    (weighted sum)
 *     LSE_i = m_i + ln l_i
 * over the valid keys j of row i, where m_i is the row maximum and l_i the
 * sum of the shifted exponentials. The definition is §2.2-§2.4 of the chapter
 * "2. 自注意力机制算子：QKV投影、注意力分数计算、Softmax、加权求和，以及FlashAttention
 * 优化"; the fused evaluation (tiles, running max and sum, rescale of the
 * partial output by exp(m_old - m_new)) is its §2.6 and the section
 * "FlashAttention 分块计算原理与浏览器适配" of "WebGPU 算子优化：QKV 内存合并与
 * FlashAttention 分块计算". The score and probability matrices never reach
 * device memory in attn_fwd / attn_fwd_splitk.
 *
 * Valid keys. Key j is valid for query i of sequence b iff j < n_b and, when
 * `causal` is nonzero, j <= i (key j > query i is masked, counted from the
 * first query and the first key, also when Sq != Sk). n_b = kv_len[b] clamped
 * to [0, Sk], or Sk when kv_len is NULL. Rows with no valid key give O = 0
 * and LSE = -inf. Key/value rows at or beyond n_b are never read.
 *
 * Tensors (all device memory, owned by the caller, never retained):
 *   q, o   [B, H, Sq, d] (ATTN_LAYOUT_BHSD) or [B, Sq, H, d] (ATTN_LAYOUT_BSHD),
 *          dense, element type `dtype`; o has the layout and type of q.
 *   k, v   the same layout with Sk rows.
 *   lse    float32 [B, H, Sq] whatever the layout, or NULL to skip it.
 *   kv_len int32 [B] or NULL.
 * The two layouts are the "Contiguous" and head-"Interleaved" QKV layouts of
 * the section "QKV 矩阵的内存合并模式选择" of the WebGPU page, read as
 * separate q, k, v tensors with heads outermost or interleaved per token;
 * its "Split" layout is ATTN_LAYOUT_SPLIT(g) below.
 * q, k, v, o and workspaces must be 16-byte aligned; lse and kv_len 4-byte.
 *
 * Arithmetic: bf16/fp16 inputs use bf16/fp16 matrix-core products with fp32
 * accumulation; the softmax state is fp32; probabilities are rounded to the
 * input type (nearest-even) before the second product; the output is rounded
 * once to the input type. fp32 inputs keep every step in fp32.
 *
 * Inputs must be finite. The kernels are compiled on the assumption that no
 * NaN occurs (a maximum of a NaN and a number may return either), and a NaN
 * or infinity in q, k or v inside the valid keys gives an undefined result:
 * it may poison the whole output row, also where exact arithmetic would give
 * that key zero weight (0 * inf). Key/value rows past kv_len are never read,
 * so they may hold anything.
 *
 * Execution: every call validates all arguments on the host first and
 * returns an error status without touching the GPU when one is bad. On
 * success it enqueues its kernels on `stream` (a hipStream_t; NULL is the
 * null stream) and returns without synchronising; outputs are valid once the
 * stream has reached that point. Launch failures return ATTN_E_HIP. The
 * library holds no state and is safe to call from several threads; calls
 * that share a workspace must be ordered by the caller.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_E_NULLPTR = 1,     /* a required pointer is NULL                        */
    ATTN_E_SHAPE = 2,       /* B, H, Sq or Sk < 1, n_split < 1, or sizes overflow */
    ATTN_E_UNSUPPORTED = 3, /* d not 64/128, enum out of range, group not dividing H */
    ATTN_E_ALIGN = 4,       /* a pointer is not aligned as stated above          */
    ATTN_E_WORKSPACE = 5,   /* workspace / scratch NULL or smaller than required */
    ATTN_E_HIP = 6,         /* the HIP runtime reported an error at launch       */
    ATTN_E_ARG = 7,         /* scale negative, NaN or infinite; tile out of range;
                             * n_split < 1 in attn_fwd_tiled                   */
    ATTN_E_SCRATCH_LIMIT = 8 /* attn_fwd_noalloc: the plan needs more workspace
                              * than ATTN_NOALLOC_SCRATCH_BYTES                */
};

enum attn_layout { ATTN_LAYOUT_BHSD = 0, ATTN_LAYOUT_BSHD = 1 };

/* The "Split" head-group layout of the same section: heads in groups of g,
 * each group's rows stored together, [B, H/g, S, g, d]. g must divide H.
 * g = 1 is the same memory order as ATTN_LAYOUT_BHSD, g = H as
 * ATTN_LAYOUT_BSHD. Accepted wherever a layout is. */
#define ATTN_LAYOUT_SPLIT(g) (0x10000 | (g))

enum attn_dtype { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 };

/*
 * Fused forward. Follows attn_fwd_plan: one fused kernel (prefill shapes),
 * the fused kernel over key ranges plus a merge (few query tiles over long
 * keys, 16-bit types), or the split-over-keys pair of kernels (one query row
 * over many keys). A plan with key splits needs `workspace` of at least
 * attn_fwd_workspace_size bytes (NULL / 0 is fine when that size is 0).
 * scale must be finite and >= 0 (0 gives uniform weights over the valid keys).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
             int dtype, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * attn_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, plan, kernels and results, without the workspace
 * arguments. Where attn_fwd's plan needs a workspace, this call uses a
 * static device buffer of the library instead: ATTN_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, held from the first such call on that GPU until the
 * process ends. A plan that needs more (attn_fwd_workspace_size above the
 * limit) returns ATTN_E_SCRATCH_LIMIT without launching anything. The call
 * allocates nothing, neither device nor pinned memory; its first call on a
 * GPU that needs the buffer looks up the buffer's address there (a HIP
 * symbol query, made with that GPU current) and keeps it.
 * All calls on one GPU share that buffer: calls whose plans use it and that
 * may overlap on that GPU (other streams, other threads without ordering)
 * race and give wrong results. Calls ordered on one stream are safe; no
 * clearing is needed between them.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                     int dtype, const int32_t* kv_len, void* stream);

/* Bytes of workspace attn_fwd needs for this shape (0 when it plans no split).
 * Returns 0 for arguments attn_fwd would reject. Host only. */
size_t attn_fwd_workspace_size(int B, int H, int Sq, int Sk, int d, int dtype, int causal);

/* The number of key splits attn_fwd will use for these arguments. The keys
 * a row can see count (with causal masking, at most Sq of them). 1: the
 * fused kernel alone. More, with one query per head: the split-over-keys
 * pair (a single query per head that sees at least 1024 keys always
 * splits). More, with two or more queries per head (fp16/bf16 only): the
 * fused kernel over key ranges, used when its (batch, head, 128-query tile)
 * workgroups number fewer than 256 and a row sees at least 4096 keys, with
 * about 512 workgroups in all, at least 1024 keys per range and at most 64
 * ranges.
 * Host only; returns a status and writes *n_split on success. */
int attn_fwd_plan(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int* n_split);

/*
 * Tile variants of the fused kernel. The WebGPU page's section
 * "浏览器端落地的关键参数与监控" picks the sequence and head-dimension tiles
 * per device by a probe at the first run, falling back to smaller tiles. Here
 * the candidates are compiled in, and the choice is a table made offline by
 * timing every candidate on the GPU over a grid of query-row counts
 * (B*H*Sq) and key lengths, per head size and masking (the package's
 * autotune script writes it; the library must be rebuilt to use a new one).
 * attn_fwd uses the table's choice for the fused kernel over all keys, and
 * one fixed variant for the fused kernel over key ranges.
 */
typedef struct attn_tile_info {
    int rows;      /* query rows per workgroup                              */
    int keys;      /* keys per tile of the LDS ring                         */
    int waves;     /* 64-lane waves per workgroup                           */
    int stages;    /* LDS ring stages                                       */
    int lds_bytes; /* LDS per workgroup                                     */
} attn_tile_info;

/* Number of tile variants for (d, dtype); 0 when the pair is unsupported.
 * Host only. */
int attn_fwd_tile_count(int d, int dtype);

/* Describe variant `tile` (0 <= tile < attn_fwd_tile_count) in *info.
 * Returns ATTN_E_NULLPTR, ATTN_E_UNSUPPORTED for a bad d or dtype, ATTN_E_ARG
 * for a tile out of range. Host only. */
int attn_fwd_tile_info(int d, int dtype, int tile, attn_tile_info* info);

/* The variant attn_fwd's fused kernel runs for this shape, in *tile: the
 * table's pick, or, where attn_fwd_plan gives the fused kernel key ranges,
 * the variant for key ranges (attn_fwd_tiled with tile -1 makes the same
 * choice for its n_split). Host only. */
int attn_fwd_tile_choice(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int* tile);

/*
 * The fused kernel with tile variant `tile` (-1: attn_fwd's choice) and
 * n_split key ranges, whatever the shape; never the split-over-keys pair.
 * n_split = 1: one kernel, no workspace (NULL / 0). n_split > 1 (fp16/bf16
 * only, else ATTN_E_UNSUPPORTED): the keys are cut into n_split ranges of
 * whole 64-key tiles (ceil(Sk / (64 n_split)) * 64 keys each; trailing
 * ranges may be empty). Each (batch, head, query tile, range) workgroup
 * writes, per query row, the unnormalised record of its range (running max,
 * running sum, weighted sum of V) to `workspace`, which must hold
 * attn_splitk_workspace_size(B, H, Sq, d, n_split) bytes, 16-byte aligned;
 * the merge kernel of attn_fwd_splitk then combines the ranges by the block
 * rule (the WebGPU page's FlashAttention section, §2.6 of the chapter).
 * Same arguments and results as attn_fwd otherwise; a tile out of range or
 * n_split < 1 is ATTN_E_ARG. For tuning and testing every variant.
 */
int attn_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                   int dtype, const int32_t* kv_len, int tile, int n_split, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * Split-over-keys forward with an explicit split count (the single-query
 * decode path). The keys [0, Sk) are cut into n_split equal ranges; each
 * (b, h, i, split) writes its unnormalised partial (running max, running
 * sum, weighted sum of V) to the workspace, and a second kernel merges the
 * partials of each row with weights exp(m_s - max_s m_s) — the block merge of
 * the WebGPU page's FlashAttention section and §2.6 of the chapter. Splits
 * with no valid key contribute nothing. Any n_split >= 1 is accepted.
 */
int attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                    int dtype, const int32_t* kv_len, int n_split, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Workspace bytes for attn_fwd_splitk (0 for rejected arguments). Host only. */
size_t attn_splitk_workspace_size(int B, int H, int Sq, int d, int n_split);

/*
 * Unfused baseline with the materialised intermediates of the chapter's §2.5:
 * kernel 1 writes S = scale * Q K^T to scratch ([B, H, Sq, Sk] in fp32, rows
 * padded to a multiple of 64 keys), kernel 2 runs the three-step softmax on
 * each row (max, then sum, then normalise, each a pass over the stored row)
 * and writes P (same shape, input type) plus LSE, kernel 3 computes O = P V.
 * Same arguments and results as attn_fwd; `scratch` must hold
 * attn_naive_scratch_size bytes.
 */
int attn_fwd_naive(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                   int dtype, const int32_t* kv_len, void* scratch, size_t scratch_bytes,
                   void* stream);

/* Scratch bytes for attn_fwd_naive: S in fp32 and P in dtype, B*H*Sq rows of
 * Sk rounded up to 64 each (0 for rejected arguments). Host only. */
size_t attn_naive_scratch_size(int B, int H, int Sq, int Sk, int dtype);

/*
 * QKV projection (§2.1 of the chapter: the three projections as one product
 * with the weights side by side, then split). For t = 0, 1, 2 it writes
 *     out_t[b, h, s, c] = sum_i x[b, s, i] * W[i, t*H*d + h*d + c]
 * to out_0 = q, out_1 = k, out_2 = v, where W is the D x 3Hd concatenation
 * [W_Q | W_K | W_V]. Storage:
 *   x      [B, S, D] dense, element type `dtype`.
 *   w      [3*H*d, D] dense: w[n*D + i] = W[i, n] (out-major, the storage of
 *          a linear layer's weight), element type `dtype`.
 *   q,k,v  [B, H, S, d] (ATTN_LAYOUT_BHSD), [B, S, H, d] (ATTN_LAYOUT_BSHD) or
 *          [B, H/g, S, g, d] (ATTN_LAYOUT_SPLIT(g)), dense, element type
 *          `dtype`: the inputs attn_fwd takes.
 * dtype is ATTN_F16 or ATTN_BF16 (fp32 returns ATTN_E_UNSUPPORTED); products
 * accumulate in fp32 and each output is rounded once (nearest-even).
 * Requirements: B, S >= 1 (else ATTN_E_SHAPE); D a positive multiple of 64
 * and d a positive multiple of 8 (else ATTN_E_SHAPE); B*S, 3*H*d and D each
 * below 2^31; all pointers 16-byte aligned (ATTN_E_ALIGN); none NULL
 * (ATTN_E_NULLPTR). Asynchronous on `stream` like attn_fwd; no workspace.
 */
int attn_qkv_proj(const void* x, const void* w, void* q, void* k, void* v, int B, int S, int D,
                  int H, int d, int layout, int dtype, void* stream);

/*
 * Which of the two tilings attn_qkv_proj runs for B*S tokens and 3*H*d
 * output columns on a GPU with n_cu compute units (attn_qkv_proj uses the
 * current device's count): 0 = 128 tokens x 192 columns per workgroup, two
 * workgroups per CU; 1 = 256 x 256, one per CU, taken when it needs clearly
 * fewer rounds of workgroups over the CUs (large products). Writes it to
 * *tiling. B, S, H, d, n_cu >= 1 (else ATTN_E_SHAPE); tiling non-NULL (else
 * ATTN_E_NULLPTR). Host only, for tests and tuning.
 */
int attn_qkv_proj_tiling(int B, int S, int H, int d, int n_cu, int* tiling);

/*
 * Row softmax: for each row r of x [rows, n],
 *     y[r, j] = exp(scale*x[r, j] - m_r) / l_r,   lse[r] = m_r + ln l_r,
 * with m_r the row maximum of scale*x and l_r the sum of the shifted
 * exponentials (§2.3 of the chapter). Entries equal to -inf get probability 0;
 * a row with no finite entry gives y = 0 and lse = -inf. This is the
 * computation the page "[Performance] [WebGPU] Proposal: Add an option to use
 * online softmax instead of naive softmax" studies on its own, in its two
 * forms, selected by `mode`:
 *   ATTN_SOFTMAX_ONLINE     the online form: a running max and a running sum
 *                           rescaled as the max grows (§四 of that page). Rows
 *                           of up to 32768 elements are read from memory once
 *                           (held on chip); longer rows twice.
 *   ATTN_SOFTMAX_THREE_PASS the naive form: separate passes for the max, the
 *                           sum and the normalisation, each reading the row.
 * Storage: x and y dense [rows, n] of `dtype` (any of the three), y may not
 * alias x; lse float32 [rows] or NULL. n must be a multiple of 8 for 16-bit
 * types and of 4 for fp32 (16-byte rows); 1 <= rows < 2^31 (ATTN_E_SHAPE);
 * scale finite and >= 0 (ATTN_E_ARG; 0 gives uniform rows over the finite
 * entries); x, y 16-byte and lse 4-byte aligned (ATTN_E_ALIGN). fp32
 * arithmetic, base-2 exponentials; y is rounded once to `dtype`.
 * Asynchronous on `stream` like attn_fwd; no workspace.
 */
enum attn_softmax_mode { ATTN_SOFTMAX_ONLINE = 0, ATTN_SOFTMAX_THREE_PASS = 1 };

int attn_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int n, float scale,
                      int dtype, int mode, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
