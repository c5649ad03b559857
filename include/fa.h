/*
 * fa.h -- C ABI of the MI355X (gfx950) IO-aware exact attention library
 * (libfa.so).
 *
 * The operation is exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * computed the IO-aware way: the N x N score and probability matrices live
 * only on chip, tile by tile, with an online softmax, and only O plus one
 * log-sum-exp per query row are written back. The backward pass recomputes
 * the probabilities on chip from that log-sum-exp.
 *
 * Sources:
 *   "FlashAttention原理：从原始Attention到FlashAttention"
 *     (blog.csdn.net/qq_43527718/article/details/142302113):
 *     section 二.2 -- the standard (unfused) pipeline whose result must be
 *     reproduced exactly; section 二.5/二.6 -- tiling and blockwise softmax;
 *     section 二.7 -- query blocks in the outer loop, key/value blocks in the
 *     inner loop, fully masked blocks skipped; section 一.2 -- the softmax
 *     normalizer is stored so the backward pass can recompute attention on
 *     chip instead of reading it from HBM.
 *   "FlashAttention：优化大模型训练的内存与计算效率" (cnnetsun.cn/a/3461300):
 *     section 3.1 -- tensors shaped (batch, heads, seq_len, dim) and the
 *     is_causal switch; section 4.1 -- softmax kept in float32 under
 *     mixed precision.
 *
 * Conventions shared by every entry point:
 *   - Layout: Q, K, V, O, dO, dQ, dK, dV are contiguous row-major
 *     [B, H, N, d] device arrays of one element type (``dtype``); LSE is a
 *     contiguous [B, H, N] float32 device array. Self-attention: queries and
 *     keys share the length N.
 *   - Causal: when ``causal`` is 1, key j is hidden from query i if j > i.
 *   - LSE_i = ln(sum_j exp(scale * q_i . k_j)) over the visible keys
 *     (natural log of the scaled scores' exponential sum).
 *   - Ownership: the caller allocates and owns every buffer (device memory).
 *     The library allocates no device memory, frees nothing and keeps no
 *     pointer after returning. Inputs are read-only; outputs must not overlap
 *     any input or each other. (fa_bwd_noalloc alone uses a scratch array
 *     the library holds statically, one per GPU; see there.)
 *   - Streams: ``stream`` is a hipStream_t (NULL = the null stream). Every
 *     call only enqueues work on it and returns; the results are ready when
 *     the stream is synchronized. The returned status covers argument
 *     validation and the kernel launches; a fault inside a kernel surfaces at
 *     the caller's next synchronization.
 *   - Supported: d in {64, 128}; dtype FA_F32, FA_F16, FA_BF16; any N >= 1;
 *     B*H*N*d < 2^40 elements and N*d < 2^31. Arithmetic: products of
 *     16-bit inputs on bf16/fp16 matrix cores (fp32 matrix cores for FA_F32)
 *     with float32 accumulation; softmax statistics in float32; outputs
 *     rounded to nearest-even into ``dtype``.
 *   - Thread safety: concurrent calls on different streams are independent,
 *     except fa_bwd_noalloc calls on one GPU, which share its static scratch.
 *   - Validation (in order; the first failure is returned and nothing is
 *     enqueued): null pointers, B/H/N < 1 or dtype unknown or causal not 0/1
 *     or scale negative/non-finite -> FA_ERR_INVALID_ARG; d not supported or
 *     sizes too large -> FA_ERR_UNSUPPORTED; a pointer not 16-byte aligned
 *     -> FA_ERR_ALIGN; overlapping output/input ranges -> FA_ERR_INVALID_ARG;
 *     workspace too small -> FA_ERR_WORKSPACE (fa_bwd_noalloc: a problem
 *     too large for its static scratch -> FA_ERR_SCRATCH).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V, O, dO, dQ, dK, dV. */
typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

/* Status codes. */
enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,
  FA_ERR_UNSUPPORTED = -2,
  FA_ERR_ALIGN = -3,
  FA_ERR_WORKSPACE = -4,
  FA_ERR_HIP = -5,
  FA_ERR_SCRATCH = -6
};

/*
 * fa_fwd -- forward attention.
 *   q, k, v : [B,H,N,d] ``dtype`` inputs (device, read-only).
 *   o       : [B,H,N,d] ``dtype`` output (device).
 *   lse     : [B,H,N] float32 output (device): the per-row log-sum-exp the
 *             backward pass needs (the stored softmax normalizer of the
 *             pages' section 一.2).
 *   scale   : multiplier of Q K^T; finite and >= 0 (1/sqrt(d) usually).
 *   causal  : 0 or 1.
 *   dtype   : an fa_dtype value.
 *   stream  : hipStream_t to enqueue on.
 * One kernel: query tiles in the outer (grid) dimension, key/value tiles in
 * the inner loop, online softmax in registers; tiles above the causal
 * diagonal are never visited. bf16/fp16 shapes with too few 256-row query
 * tiles to give every compute unit one (B*H*ceil(N/256) < 256, or <= 256
 * with causal = 1, where one round of tiles is uneven) run the key-split
 * kernel of fa_fwd_keysplit instead; the results agree to float rounding.
 * Returns FA_OK or a negative status (see the conventions above).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd (and
 * fa_bwd_ex) needs: a float32 [B,H,N] row term D_i = sum_k dO_ik O_ik and
 * a float32 scratch of 2*B*H*N*d elements, each 256-byte aligned. The
 * scratch holds the dQ accumulator (FA_F32) or, with grouped K/V heads whose
 * query heads are split over several workgroups, their partial dK and dV
 * (FA_F16, FA_BF16). Returns 0 for invalid sizes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd -- backward attention for the loss sum(dO * O).
 *   q, k, v, o, dO : [B,H,N,d] ``dtype`` (device, read-only); o is the
 *                    forward output.
 *   lse            : [B,H,N] float32 from fa_fwd (device, read-only).
 *   dq, dk, dv     : [B,H,N,d] ``dtype`` outputs (device).
 *   workspace      : device scratch of at least fa_bwd_workspace_size()
 *                    bytes, 256-byte aligned, owned by the caller; its
 *                    contents on entry are ignored (the library clears what
 *                    it needs on ``stream``) and undefined on exit.
 *   other arguments as for fa_fwd (scale and causal must match the forward).
 * The probabilities are recomputed on chip from Q, K and LSE (never read
 * from memory). bf16/fp16: dK and dV come from a kernel with key tiles as
 * the outer (grid) dimension and query tiles in the inner loop, dQ from a
 * kernel with query tiles outer and key tiles inner; no atomics, so the
 * results repeat bit for bit. float32: one key-outer kernel that adds dQ
 * into a float32 accumulator in the workspace.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dO, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, results
 * and kernels as fa_bwd, except that the scratch (the float32 row term D,
 * and for FA_F32 the float32 dQ accumulator) lives in the library's own
 * static device array of 64 MiB, one per GPU, held until the process ends.
 * Nothing is allocated or freed by the call.
 *   Limit: 4*B*H*N bytes (bf16, fp16) or 4*B*H*N*(d+1) bytes (FA_F32), each
 *   part rounded up to 256, must fit in 64 MiB; larger problems return
 *   FA_ERR_SCRATCH before anything is enqueued (use fa_bwd with a workspace).
 *   Concurrency: every call on one GPU uses that GPU's one array, so calls
 *   that overlap in time on one GPU (different streams, or threads) race and
 *   must be serialized by the caller; calls in one stream are ordered. The
 *   array keeps the last call's contents; each call writes what it reads
 *   before reading it (D, and the zeroed accumulator for FA_F32) with
 *   kernels on ``stream`` (no memset nodes).
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   void* stream);

/*
 * Variants: grouped K/V heads and local windows.
 *
 * fa_options selects two generalizations of the operation above. Both
 * reduce to it with kv_heads = 0 (or H) and both window bounds negative.
 *   kv_heads     : Hkv, the number of K/V heads (multi-query / grouped-query
 *                  attention). It must divide H; 0 means H. K, V (and in the
 *                  backward dK, dV) are then [B, Hkv, N, d]. Query head h
 *                  attends with K/V head h / (H / Hkv), and dK, dV of a K/V
 *                  head are the sums over the query heads that use it.
 *   window_left  : >= 0: key j is hidden from query i if j < i - window_left.
 *                  Negative: no bound on that side.
 *   window_right : >= 0: key j is hidden from query i if j > i + window_right.
 *                  Negative: no bound on that side. The window combines with
 *                  ``causal`` (causal alone is the window (unbounded, 0)).
 * A bound of N - 1 or more hides no key on its side and is treated as
 * unbounded, so every int value is accepted for either bound.
 * Every query row sees at least its own key (a non-negative bound never
 * excludes j = i). Key tiles that lie entirely outside every query's window
 * are never visited: they generalize the causal tile skipping of the pages'
 * section 二.7 to a band.
 */
typedef struct fa_options {
  int kv_heads;
  int window_left;
  int window_right;
} fa_options;

/*
 * fa_fwd_ex -- fa_fwd with options (``opts`` may be NULL: plain attention).
 * k and v are [B, Hkv, N, d]; everything else as for fa_fwd. Validation adds:
 * kv_heads < 0, or not dividing H -> FA_ERR_INVALID_ARG.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              const fa_options* opts, void* stream);

/*
 * fa_fwd_keysplit -- fa_fwd_ex computed by the key-split kernel, whatever
 * the shape (fa_fwd and fa_fwd_ex choose it by themselves for small grids).
 * A workgroup covers 64 query rows (d = 64) or 128 (d = 128); its key tiles
 * are dealt out over 4 (d = 64) or 2 (d = 128) groups of its waves, each of
 * which runs the online softmax over its own tiles, and the groups' partial
 * (O, max, sum) are combined in LDS at the end: the blockwise softmax merge
 * of the pages' sections 二.5/二.6 within one workgroup. It shortens the
 * chain of key tiles behind each output row, for sequences whose query tiles
 * are too few to fill the GPU, without the float32 partials and second
 * launch of fa_fwd_splitkv. bf16 and fp16 only: FA_F32 returns
 * FA_ERR_UNSUPPORTED. Arguments, validation and results otherwise as for
 * fa_fwd_ex.
 */
int fa_fwd_keysplit(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, int dtype,
                    const fa_options* opts, void* stream);

/*
 * fa_bwd_ex -- fa_bwd with options (``opts`` may be NULL). k, v, dk, dv are
 * [B, Hkv, N, d]; the workspace size is fa_bwd_workspace_size(B, H, N, d)
 * (it depends on the query heads only). scale, causal and opts must match
 * the forward call that produced o and lse.
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
              const void* dO, const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              const fa_options* opts, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Split-KV forward.
 *
 * fa_fwd launches one workgroup per query tile of every head, so a short
 * sequence with few heads leaves most compute units idle. fa_fwd_splitkv
 * also splits the key tiles each query tile visits into ``num_splits``
 * contiguous slices, one workgroup each. A slice's workgroup runs the same
 * online softmax over its keys only and writes a float32 partial: O
 * normalized over those keys, and their LSE (-inf for a row that sees none
 * of them). A second kernel then merges the partials of each row with
 * M = max_s LSE_s and w_s = exp(LSE_s - M): O = sum_s w_s O_s / sum_s w_s,
 * LSE = M + ln(sum_s w_s). This is the blockwise softmax combination of the
 * pages' sections 二.5/二.6, taken across workgroups instead of across the
 * steps of one loop; the results equal fa_fwd_ex's up to float rounding.
 */

/*
 * fa_fwd_num_splits -- the slice count fa_fwd_splitkv uses when called with
 * num_splits = 0: the smallest power of two (at most 16) that gives every
 * compute unit a workgroup, while each slice keeps at least four 64-key
 * tiles. 1 means no split. Returns 0 for invalid sizes or dtype.
 */
int fa_fwd_num_splits(int B, int H, int N, int d, int dtype);

/*
 * fa_fwd_splitkv_workspace_size -- bytes of device workspace fa_fwd_splitkv
 * needs with ``num_splits`` slices (0: the count fa_fwd_num_splits picks):
 * float32 partial outputs [S, B, H, N, d] and partial LSE [S, B, H, N],
 * each 256-byte aligned. 0 when S is 1 (no workspace is used) or for
 * invalid arguments.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int N, int d, int dtype, int num_splits);

/*
 * fa_fwd_splitkv -- fa_fwd_ex computed with split-KV (see above).
 *   num_splits : 1..64 slices, or 0 for fa_fwd_num_splits' choice. With 1
 *                there is no split and no merge: the row-tiled kernel alone
 *                (one workgroup per 256 query rows; 128 for FA_F32), which
 *                is what fa_fwd_ex runs for shapes that fill the GPU.
 *   workspace  : device scratch of at least fa_fwd_splitkv_workspace_size()
 *                bytes for the same arguments, 256-byte aligned, owned by the
 *                caller; contents on entry are ignored and undefined on exit.
 *                May be NULL when that size is 0.
 *   other arguments as for fa_fwd_ex (opts may be NULL).
 * Validation adds: num_splits outside 0..64 -> FA_ERR_INVALID_ARG; workspace
 * NULL or too small while one is needed -> FA_ERR_WORKSPACE; workspace
 * overlapping an input or output -> FA_ERR_INVALID_ARG.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   const fa_options* opts, int num_splits, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * 8-bit float forward.
 *
 * The pages list lower-precision data types (FP8, INT8) among the method's
 * next steps (section "应用展望" of "FlashAttention与新一代硬件架构融合：
 * 解锁大模型训练新高度") without a
 * scheme. This entry point reads Q, K and V as OCP FP8 E4M3 codes (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F and 0xFF
 * are NaN; largest finite value 448), each tensor with one dequantization
 * factor, and computes the attention of fa_fwd_ex over the values those
 * codes stand for:
 *   Q = q_descale * Q8, K = k_descale * K8, V = v_descale * V8,
 *   O = softmax(scale * Q K^T [causal rule, window]) V,  LSE as for fa_fwd.
 * The score products and the P V product run on the gfx950 FP8 matrix cores
 * with float32 accumulation; the softmax is float32 and its probabilities
 * enter the P V product as E4M3 codes (relative rounding 2^-4 each), the
 * normalizer and LSE are taken from the unrounded values. See the parity
 * tests for the error bound this implies.
 *
 * fa_fwd_fp8
 *   q        : [B, H, N, d] E4M3 codes (one byte each), device memory.
 *   k, v     : [B, Hkv, N, d] E4M3 codes (Hkv from opts->kv_heads, default H).
 *   o        : [B, H, N, d] output in ``out_dtype`` (FA_BF16 or FA_F16).
 *   lse      : [B, H, N] float32 output, natural log.
 *   q_descale, k_descale, v_descale : finite, > 0.
 *   scale    : softmax scale, finite, >= 0 (the scores use
 *              scale * q_descale * k_descale, which must be finite).
 *   causal, opts, stream : as for fa_fwd_ex (opts may be NULL).
 * All pointers 16-byte aligned; outputs must not overlap inputs or each
 * other. Inputs must not hold NaN codes (a NaN anywhere in a visited tile
 * can reach every row of that tile). The result for every row is written;
 * nothing is allocated. Status: as fa_fwd_ex, plus out_dtype not FA_BF16 or
 * FA_F16 -> FA_ERR_INVALID_ARG (FA_F32 -> FA_ERR_UNSUPPORTED), a descale
 * not finite and positive -> FA_ERR_INVALID_ARG.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float q_descale, float k_descale, float v_descale, int out_dtype,
               const fa_options* opts, void* stream);

/*
 * Block-sparse attention.
 *
 * The pages name block-sparse attention among the method's extensions
 * (section 6.1 "稀疏注意力变体" of "FlashAttention：优化大模型训练的内存与计算
 * 效率") without fixing a format. Here the pattern is a map over blocks of
 * FA_MASK_BLOCK query rows by FA_MASK_BLOCK keys: with nmb = ceil(N / 64),
 * block_mask is a row-major [nmb, nmb] array of bytes in device memory, the
 * same for every batch and head, and
 *   key j is hidden from query i  if  block_mask[i / 64][j / 64] == 0,
 * on top of the causal rule, the window and grouped heads of fa_options. The
 * kernels never visit a key tile that every query row of a workgroup has
 * dropped, as the pages' section 二.7 skips the tiles above the causal
 * diagonal. A query row that sees no key at all gets O = 0 and LSE = -inf,
 * and its gradient terms are 0 (dQ = 0; it adds nothing to dK or dV).
 *
 * fa_fwd_sparse -- fa_fwd_ex under a block mask.
 * fa_bwd_sparse -- fa_bwd_ex under the same block mask (scale, causal, opts
 *                  and block_mask must match the forward call that produced
 *                  o and lse).
 *   block_mask : [nmb, nmb] bytes, device memory, read-only, owned by the
 *                caller; no alignment needed; it must not overlap any output
 *                or the workspace.
 *   other arguments as for fa_fwd_ex / fa_bwd_ex.
 * Status: as fa_fwd_ex / fa_bwd_ex, plus block_mask NULL or overlapping an
 * output -> FA_ERR_INVALID_ARG; dtype FA_F32 or N > 65536 (nmb > 1024)
 * -> FA_ERR_UNSUPPORTED.
 */
#define FA_MASK_BLOCK 64

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const fa_options* opts, const void* block_mask, void* stream);

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse, void* dq, void* dk, void* dv,
                  int B, int H, int N, int d, float scale, int causal, int dtype,
                  const fa_options* opts, const void* block_mask, void* workspace,
                  size_t workspace_bytes, void* stream);

/* fa_strerror -- static, NUL-terminated description of a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
