/*
 * wan_attn.h -- C ABI of the MI355X (gfx950) attention forward for Wan video DiT blocks (and of the
 * attention backward, the FP8 GEMM of the DiT linear layers and block-sparse attention, declared
 * further below).
 *
 * Operation (every entry point below computes it, or a stage of it):
 *   O[b, i, h, :] = sum_j softmax_j( Q[b,i,h,:] . K[b,j,h,:] / sqrt(head_dim) ) * V[b, j, h, :]
 * non-causal and unmasked: the full spatio-temporal self-attention over the video tokens of a Wan
 * DiT block, and its cross-attention to the 512 umT5 text tokens ("Wan 2.1: VBench 86.22% ..."
 * explainer of the Wan technical report, sections "先看现象" -- non-causal attention, forward cost
 * beta = 4 in C = L(alpha*b*s*h^2 + beta*b*s^2*h) -- and "干预与形式化", DiT backbone paragraph).
 * The scale is fixed at 1/sqrt(head_dim); there is no mask argument.
 *
 * Layouts (all entry points): row-major, dense, contiguous, device memory
 *   q, o : [batch, s_q,  heads, head_dim]  bfloat16
 *   k, v : [batch, s_kv, heads, head_dim]  bfloat16
 * head_dim must be 128; heads <= 65536.  Pointers must be 16-byte aligned.  o must not overlap
 * q, k or v.
 *
 * Ownership: the caller owns every buffer it passes; the library never frees or retains them.
 * Streams: every call only enqueues work on `stream` (a hipStream_t; NULL is the default stream)
 * and returns; results are ready when the stream reaches that point.  A fault inside a kernel
 * surfaces at the caller's next synchronisation, not in the return code.
 * Errors: every function returns WAN_ATTN_OK (0) or a negative code below; it never aborts and
 * never prints unless the environment variable WAN_ATTN_LOG=1 is set.  Argument checks happen
 * before any work is enqueued, so a failed check leaves the stream untouched.
 * Scratch memory: the entry points that need scratch take it from a per-device stream-ordered pool
 * of the library (allocated and freed on the caller's stream).  Freed scratch stays in the pool
 * for the next call (the largest call's scratch is kept for the life of the process) until
 * wan_attn_release_scratch() returns it to the driver.  Test hook: if the environment variable
 * WAN_ATTN_TEST_FAIL_ALLOC=1 is set when the library first needs scratch, every scratch
 * allocation of the process fails with WAN_ATTN_ENOMEM (the variable is read once).
 */
#ifndef WAN_ATTN_H
#define WAN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WAN_ATTN_VERSION 1

/* Arithmetic of the call (the `dtype` argument). */
enum wan_attn_dtype {
  /* bf16 x bf16 MFMA products with fp32 accumulation, fp32 online softmax, bf16 output. */
  WAN_ATTN_BF16 = 0,
  /* The 8-bit scheme of the Wan inference optimisations ("Wan 2.1: VBench 86.22% ..." explainer,
   * section "干预与形式化"; "Wan模型是什么它能做什么" explainer, section 4.2): Q and K in int8 for
   * QK^T, P and V in FP8 (OCP e4m3) for PV, fp32 accumulation across KV blocks.  The library
   * quantises the bf16 inputs itself (see wan_attn8_quantize) into stream-ordered scratch memory
   * it allocates and frees on `stream`.  Output is bf16. */
  WAN_ATTN_INT8_FP8 = 1
};

/* Return codes. */
enum wan_attn_status {
  WAN_ATTN_OK = 0,
  WAN_ATTN_EINVAL = -1,        /* null pointer, non-positive size, unknown dtype, overflow   */
  WAN_ATTN_EALIGN = -2,        /* a pointer is not 16-byte aligned                            */
  WAN_ATTN_ENOMEM = -3,        /* scratch allocation failed                                   */
  WAN_ATTN_ELAUNCH = -4,       /* the HIP runtime refused a launch or a query                 */
  WAN_ATTN_EUNSUPPORTED = -5   /* head_dim other than 128; an FP8 GEMM or VSA size outside its limits */
};

/*
 * Attention forward.  q, k, v, o as in the header comment; batch, heads, s_q, s_kv >= 1;
 * head_dim == 128; dtype is a wan_attn_dtype; stream is a hipStream_t or NULL.
 * bf16: needs no scratch memory, except when batch*heads*ceil(s_q/256) is below half the GPU's
 * compute units and s_kv >= 193: then each query tile's keys are split into ranges attended in
 * parallel, and about batch*heads*ceil(s_q/256)*ranges*133 KB (ranges <= 2*CUs) of scratch is
 * allocated on `stream` and freed on `stream` after use.  int8_fp8: allocates about
 * s_q*heads*batch*(head_dim+4) + s_kv*heads*batch*(2*head_dim+4) bytes of scratch on `stream`,
 * freed on `stream` after use.  WAN_ATTN_ENOMEM when a scratch allocation fails.  int8_fp8 also
 * needs 128 * ceil(s_kv/64)*64 < 2^31 (s_kv up to 16,777,152; else WAN_ATTN_EUNSUPPORTED).
 */
int wan_attn_fwd(const void* q, const void* k, const void* v, void* o,
                 int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                 int64_t head_dim, int dtype, void* stream);

/*
 * First stage of the 8-bit path, exposed so that its integer outputs can be checked code for
 * code and the second stage timed alone.  Inputs q, k, v as above (bf16).  Outputs, all device
 * memory owned by the caller:
 *   q_codes [batch, s_q, heads, 128] int8     k_codes [batch, s_kv, heads, 128] int8
 *   q_scale [batch, heads, ceil(s_q/64)]  f32 k_scale [batch, heads, ceil(s_kv/64)] f32
 *   v_codes [batch, heads, 128, s_kv_pad] e4m3 bytes, V transposed per head, s_kv_pad =
 *           ceil(s_kv/64)*64, zero bytes in the padding
 *   v_scale [batch, heads, 128] f32           smooth  [batch, heads, 128] f32
 * Per (batch, head): smooth[c] = sqrt(max_t|K[t,c]| / max_t|Q[t,c]|) (1 if either is 0);
 * Q' = Q*smooth, K' = K*(1/smooth) in fp32; one int8 scale per 64-token block of Q' (K') over all
 * channels: inv = 127/amax, code = clamp(rne(x*inv), -127, 127), scale = amax/127 (amax = 0:
 * codes 0, scale 1); V: one scale per channel over all tokens: inv = 448/amax,
 * code = e4m3(clamp(V*inv, +-448)) with round-to-nearest-even, scale = amax/448.
 * scratch must hold wan_attn8_quantize_scratch_bytes(batch, heads) bytes (16-byte aligned).
 * No output (scratch included) may overlap another output or an input (WAN_ATTN_EINVAL).
 */
int wan_attn8_quantize(const void* q, const void* k, const void* v,
                       int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim,
                       void* q_codes, void* q_scale, void* k_codes, void* k_scale,
                       void* v_codes, void* v_scale, void* smooth, void* scratch, void* stream);

/* Bytes of scratch wan_attn8_quantize needs (per-channel maxima of Q, K and V). */
size_t wan_attn8_quantize_scratch_bytes(int64_t batch, int64_t heads);

/*
 * Second stage of the 8-bit path: attention from the quantised operands of wan_attn8_quantize
 * (same layouts and meaning), writing o [batch, s_q, heads, 128] bf16:
 *   S = int32(q_code . k_code) * q_scale * k_scale / sqrt(128);  online softmax in fp32 over
 *   64-key blocks;  P~ = e4m3(p * 256);  O = alpha*O + P~ . V~ (fp8 MFMA, fp32 accumulation);
 *   l = alpha*l + sum p;  out = bf16(O * v_scale[c] / (256 * l)).
 * o must not overlap the codes or scales (WAN_ATTN_EINVAL); 128 * ceil(s_kv/64)*64 < 2^31
 * (WAN_ATTN_EUNSUPPORTED otherwise).
 */
int wan_attn8_fwd_quantized(const void* q_codes, const void* q_scale,
                            const void* k_codes, const void* k_scale,
                            const void* v_codes, const void* v_scale, void* o,
                            int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                            int64_t head_dim, void* stream);

/*
 * bf16 attention forward that also writes the row statistic the backward needs:
 *   lse [batch, heads, s_q] f32 (device memory, 16-byte aligned, owned by the caller),
 *   lse[b, h, i] = log( sum_j exp( Q[b,i,h,:] . K[b,j,h,:] / sqrt(128) ) )   (natural log).
 * Otherwise exactly wan_attn_fwd with dtype WAN_ATTN_BF16 (same o, same scratch rules); lse must
 * not overlap q, k, v or o.
 */
int wan_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, void* lse,
                     int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                     int64_t head_dim, void* stream);

/*
 * bf16 attention backward: the gradients of the forward above with respect to q, k and v, given
 * the upstream gradient d_o -- the beta = 8 term of the DiT cost model, the part of training that
 * attention dominates ("Wan 2.1: VBench 86.22% ..." explainer, section "先看现象").  With
 * S = Q K^T/sqrt(128), P = exp(S - lse) (row softmax), D_i = sum_c dO[i,c] O[i,c]:
 *   dV = P^T dO,   dS = P * (dO V^T - D),   dQ = dS K / sqrt(128),   dK = dS^T Q / sqrt(128)
 * per (batch, head), products in bf16 on the MFMA with fp32 accumulation, P and dS rounded to
 * bf16 for the products (the dS that feeds dK is formed from P rounded to 11 significant bits),
 * outputs rounded to bf16.
 * Inputs: q, k, v as for the forward; o [batch, s_q, heads, 128] bf16 and lse [batch, heads, s_q]
 * f32 from wan_attn_fwd_lse on the same q, k, v; d_o with o's layout.
 * Outputs: dq with q's layout, dk and dv with k's layout, bf16, owned by the caller; none may
 * overlap another output or an input.
 * Scratch: 8 * batch * heads * ceil(s_q/64)*64 bytes allocated on `stream` and freed on `stream`
 * after use (WAN_ATTN_ENOMEM if that fails).
 */
int wan_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                 const void* lse, void* dq, void* dk, void* dv,
                 int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim,
                 void* stream);

/*
 * wan_attn_bwd without any allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight training loops and harnesses that forbid hipMalloc.  Same arguments,
 * checks and results (bit for bit) as wan_attn_bwd.  Instead of pool scratch it uses a static
 * 64 MiB device array of the library (one per GPU, held until the process ends), so it needs
 * 8 * batch * heads * ceil(s_q/64)*64 <= 64 MiB, i.e. batch * heads * ceil(s_q/64)*64 <= 8,388,608
 * (Wan-14B 720p at batch 2 and 40 heads: 6,051,840), else WAN_ATTN_EUNSUPPORTED.  Its first call on
 * a device looks up that device's copy of the array.  Every call on one GPU shares the array: calls
 * that overlap in time on one GPU (on different streams, or from different threads) race and give
 * wrong gradients; calls ordered on one stream do not.  No state carries from one call to the next.
 */
int wan_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                         const void* lse, void* dq, void* dk, void* dv,
                         int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim,
                         void* stream);

/*
 * FP8 GEMM of the DiT linear layers (the alpha term of the cost model): Y = X W^T in FP8 with the
 * activations quantised per token and the weights per tensor ("Wan模型是什么它能做什么"
 * explainer, section 4.2, where every matrix multiplication of the linear layers runs this way).
 * Codes are OCP e4m3fn (max 448); for a row (activations) or the whole tensor (weights):
 *   amax = max |x|,  inv = 448 / amax,  code = e4m3fn( clamp(x * inv, -448, 448) )  (round to nearest
 *   even, the product taken in fp32),  scale = amax / 448;  amax = 0 gives inv = scale = 1.
 * Product: Y[m, n] = bf16( (sum_k X~[m, k] * W~[n, k]) * scale_x[m] * scale_w ), the products of the
 * FP8 values accumulated in fp32 on the matrix cores.  No bias.
 * Layouts: row-major, dense, device memory.  x [rows, cols] and w [rows, cols] bf16; codes uint8 with
 * the same shape; y [m, n] bf16.  Sizes: rows >= 1; cols (the reduced dimension k) a multiple of 64,
 * at most 2^20 (else WAN_ATTN_EUNSUPPORTED); for the GEMM also n a multiple of 4
 * (WAN_ATTN_EUNSUPPORTED).  Tensors and codes 16-byte aligned, scales 4-byte aligned
 * (WAN_ATTN_EALIGN).  Outputs must not overlap the inputs (WAN_ATTN_EINVAL).  No scratch memory.
 */

/* Per-token quantisation of x [rows, cols] bf16: codes [rows, cols] uint8, scales [rows] f32. */
int wan_fp8_quantize_rows(const void* x, int64_t rows, int64_t cols, void* codes, void* scales,
                          void* stream);

/* Per-tensor quantisation of w [rows, cols] bf16: codes [rows, cols] uint8 and one f32 scale at
 * `scale` (the word also holds the running amax while the call's kernels run on `stream`). */
int wan_fp8_quantize_tensor(const void* w, int64_t rows, int64_t cols, void* codes, void* scale,
                            void* stream);

/* y [m, n] bf16 = (x_codes [m, k] . w_codes [n, k]^T) * x_scales[m] * (*w_scale), as above. */
int wan_fp8_gemm(const void* x_codes, const void* x_scales, const void* w_codes, const void* w_scale,
                 void* y, int64_t m, int64_t n, int64_t k, void* stream);

/*
 * Block-sparse attention in the style of Video Sparse Attention (VSA) (the FastWan / VSA article,
 * sections "传统稀疏注意力，为何会在蒸馏中失效？" and "一张卡，秒生视频": a coarse stage picks the key
 * blocks that matter, a fine stage runs block-sparse attention over them; 64 x 64 blocks; 87.5%
 * sparsity).  Blocks are 64 consecutive tokens of the flattened sequence from token 0 (the last one
 * may be partial); n_qb = ceil(s_q/64), n_kb = ceil(s_kv/64).
 *   Coarse: per (batch, head), mean_q[i] and mean_k[j] = the fp32 means of Q and K over the real
 *   tokens of each block; score[i, j] = mean_q[i] . mean_k[j] / sqrt(128) in fp32; for every query
 *   block i the `keep` key blocks of largest score (equal scores: lower index first), listed in
 *   ascending order: block_idx [batch, heads, n_qb, keep] int32.
 *   Fine: O[b, t, h, :] = sum over the keys of the selected blocks of query block t/64 of
 *   softmax(Q . K / sqrt(128)) V, the softmax over those keys alone; bf16 products on the MFMA,
 *   fp32 accumulation and softmax, bf16 output.
 * q, k, v, o as in the header comment (bf16, 16-byte aligned; o must not overlap q, k or v).
 * keep: 1 <= keep <= n_kb (WAN_ATTN_EINVAL otherwise); n_kb <= 4096, i.e. s_kv <= 262,144
 * (WAN_ATTN_EUNSUPPORTED).
 */

/* Bytes of scratch wan_vsa_select needs: the block means, (n_qb + n_kb) * batch * heads * 512. */
size_t wan_vsa_select_scratch_bytes(int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv);

/* Coarse stage: block_idx [batch, heads, n_qb, keep] int32 (device memory, 16-byte aligned, owned by
 * the caller), from q and k.  scratch: wan_vsa_select_scratch_bytes(...) bytes, 16-byte aligned, not
 * overlapping any other argument; it holds the block means after the call. */
int wan_vsa_select(const void* q, const void* k, int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv,
                   int64_t head_dim, int64_t keep, void* block_idx, void* scratch, void* stream);

/* Fine stage for a given block list block_idx [batch, heads, n_qb, keep] int32 (any indices: an entry
 * outside [0, n_kb) is skipped, a repeated one counts twice; the rows of a query block whose list has
 * no valid entry are undefined).  No scratch memory. */
int wan_vsa_attn(const void* q, const void* k, const void* v, const void* block_idx, void* o,
                 int64_t batch, int64_t heads, int64_t s_q, int64_t s_kv, int64_t head_dim, int64_t keep,
                 void* stream);

/* Both stages.  keep <= 0 selects ceil(n_kb / 8) (87.5% sparsity).  The block list and the block means
 * live in scratch allocated and freed on `stream` (WAN_ATTN_ENOMEM if that fails). */
int wan_vsa_fwd(const void* q, const void* k, const void* v, void* o, int64_t batch, int64_t heads,
                int64_t s_q, int64_t s_kv, int64_t head_dim, int64_t keep, void* stream);

/* Returns the library's cached scratch memory (the pools of every device it has used) to the
 * driver.  Call it when no call of the library is in flight on any stream (after synchronising
 * them); later calls allocate scratch again.  WAN_ATTN_OK, or WAN_ATTN_ELAUNCH if the runtime
 * refused. */
int wan_attn_release_scratch(void);

/* Static English text for a status code (never NULL). */
const char* wan_attn_strerror(int code);

/* WAN_ATTN_VERSION of the built library. */
int wan_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WAN_ATTN_H */
