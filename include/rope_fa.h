/*
 * rope_fa.h — C ABI of librope_fa.so: rotary position embedding (RoPE) tables,
 * the standalone rotate-half RoPE of Q and K, RoPE fused into a causal
 * FlashAttention-style forward pass, the fused RMSNorm + RoPE + KV-cache write and
 * decode-step RoPE + GQA attention over that cache, for AMD Instinct MI355X (gfx950).
 *
 * Page key for the citations below (the source pages of the method):
 *   [RoPE-fusion blog]     devpress.csdn.net/awstech/6a91ac403bda720d4b352e13
 *   [FlashAttention blog]  hwcomputing.csdn.net/6a0d3f5c662f9a54cb75d0b0
 *   [DynamicNTKOperation]  hiascend.com API page ascendtb_01_0140
 *   [RoPE/GQA tutorial]    smarter.xin/posts/3494b8a4
 *
 * Conventions shared by every entry point:
 *  - Plain C types only; no exception crosses this boundary.
 *  - The caller owns every buffer, scratch space included (rope_decode_attn_fwd takes a
 *    workspace).  The library allocates no device or host memory and keeps no mutable
 *    global state; entry points are re-entrant.
 *  - Device work is enqueued on the caller's HIP stream (`hip_stream`, a
 *    hipStream_t passed as void*, NULL = the default stream) and is
 *    asynchronous: nothing here synchronizes the device.
 *  - Every argument is validated on the host before any HIP call.  On any
 *    error the call returns a non-zero rope_status, enqueues nothing and
 *    writes nothing.  An argument the kernels cannot serve (a head_dim, a
 *    stride, an alignment) is an error, never a silent fallback to another
 *    path (the [RoPE-fusion blog] and its sibling pages warn that fused
 *    operators silently falling back is the failure mode to avoid).
 *  - Device pointers must be 16-byte aligned and every row stride a multiple
 *    of 16 bytes (vectorized 16-byte accesses); otherwise ROPE_ERR_UNSUPPORTED.
 */
#ifndef ROPE_FA_H
#define ROPE_FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROPE_FA_ABI_VERSION 3

typedef enum rope_status {
    ROPE_OK = 0,
    ROPE_ERR_NULL = 1,         /* a required pointer is NULL */
    ROPE_ERR_SHAPE = 2,        /* non-positive or inconsistent sizes */
    ROPE_ERR_DTYPE = 3,        /* dtype UNDEFINED, unknown, or not allowed for this argument */
    ROPE_ERR_LIMIT = 4,        /* a documented size limit is exceeded */
    ROPE_ERR_UNSUPPORTED = 5,  /* well-formed but not served by the kernels (head_dim, stride, alignment) */
    ROPE_ERR_ABI = 6,          /* struct_size mismatch or reserved bytes not zero */
    ROPE_ERR_HIP = 7,          /* the HIP runtime reported an error for a launch */
    ROPE_ERR_WORKSPACE = 8     /* the caller's workspace is missing, misaligned or too small */
} rope_status;

/* Element types.  UNDEFINED is never valid ([DynamicNTKOperation], 参数列表:
 * outDataType defaults to an unusable UNDEFINED that the caller must replace). */
typedef enum rope_dtype {
    ROPE_DT_UNDEFINED = 0,
    ROPE_DT_F16 = 1,
    ROPE_DT_BF16 = 2,
    ROPE_DT_F32 = 3
} rope_dtype;

/* Which coordinates form the 2-D pairs that RoPE rotates (pair i turns by angle
 * theta_i = position * inv_freq[i]).
 *   HALF:        pair i = (x[i], x[i + D/2]); tables hold theta_i in columns i and i + D/2
 *                (emb = cat(freq, freq), [DynamicNTKOperation], 算子功能分析).
 *   INTERLEAVED: pair i = (x[2i], x[2i + 1]) (the adjacent 2-D blocks of the [RoPE/GQA
 *                tutorial], section 六); tables hold theta_i in columns 2i and 2i + 1.
 * Either way the rotation of a pair (a, b) is a' = a*cos - b*sin, b' = b*cos + a*sin,
 * each output using the table values of its own column. */
typedef enum rope_pairing {
    ROPE_PAIR_HALF = 0,
    ROPE_PAIR_INTERLEAVED = 1
} rope_pairing;

/* How table angles are formed.
 *   F32:   fl32(fl32(pos / pos_scale) * inv_freq) and float32 sin/cos (the table op's own
 *          input types, int32 positions and float32 inverse frequencies).
 *   EXACT: (pos / pos_scale) * inv_freq and sin/cos in float64, rounded once to the output
 *          type: no float32 angle rounding, whose error grows with the position. */
typedef enum rope_angle_mode {
    ROPE_ANGLE_F32 = 0,
    ROPE_ANGLE_EXACT = 1
} rope_angle_mode;

/* Limits of the table op ([DynamicNTKOperation], 约束说明). */
#define ROPE_MAX_HEAD_SIZE 2048   /* head_size <= 2048 and a multiple of 32 */
#define ROPE_MAX_BATCH 16         /* batch <= 16 */
#define ROPE_MAX_NTOKENS 256000   /* ntokens <= 256000 */

/*
 * rope_inv_freq — host-side inverse frequencies, one row per sequence.
 *
 * out[b, i] = fl32(1 / base_b ** (2i / head_size)), i < head_size/2
 * ([RoPE-fusion blog], section 1.2: frequency i is 1 / base^(2i/D) for even indices 2i < D),
 * formed in double precision and rounded once to float.
 * base_b = base when trained_len <= 0 or seq_lens[b] <= trained_len; otherwise the
 * dynamic-NTK enlarged base base * (seq_lens[b] / trained_len) ** (D / (D - 2))
 * ([DynamicNTKOperation], 功能说明: no interpolation up to the trained length, base
 * enlarged above it; the page's own enlargement formula is lost, this law is the
 * reading taken).
 *
 *   base       > 0 and finite.
 *   head_size  even, 2..ROPE_MAX_HEAD_SIZE.
 *   seq_lens   HOST [batch] int32, each > 0; may be NULL only when trained_len <= 0.
 *   batch      1..ROPE_MAX_BATCH.
 *   out        HOST [batch, head_size/2] float, row-major, written by the call.
 * Pure host computation; no HIP call.  Errors: NULL, SHAPE, LIMIT.
 */
rope_status rope_inv_freq(double base, int32_t head_size, const int32_t* seq_lens, int32_t batch,
                          int32_t trained_len, float* out);

/*
 * rope_tables — the cos/sin tables of the DynamicNTK op ([DynamicNTKOperation],
 * 算子功能分析): for each sequence b and each of its tokens t,
 *   freq[t, i] = fl32(fl32(pos[t] / pos_scale) * inv_freq[b, i]),   i < head_size/2
 *   sin_out[t, j] = sin(freq[t, j mod head_size/2]),  cos_out[t, j] = cos(freq[t, j mod head_size/2])
 * (each angle fills column j and column j + head_size/2), rounded to nearest-even into out_dtype (fp16 subnormals kept).  pos_scale is the
 * linear rope_scaling_factor of the [RoPE-fusion blog], section 5.3 (positions are
 * divided by it before the outer product; 1.0f = no scaling).
 *
 *   pos        DEVICE [ntokens] int32, packed sequence after sequence ([DynamicNTKOperation],
 *              输入: positionIds restart at 0 for each batch; any int32 value is accepted).
 *   inv_freq   DEVICE [batch, head_size/2] float, row-major (row b serves sequence b).
 *   seq_lens   HOST [batch] int32, each > 0, sum == ntokens.
 *   batch      1..ROPE_MAX_BATCH;  ntokens 1..ROPE_MAX_NTOKENS;
 *   head_size  multiple of 32, 32..ROPE_MAX_HEAD_SIZE.
 *   pos_scale  finite and > 0.
 *   out_dtype  ROPE_DT_F16 or ROPE_DT_BF16 (the page's two choices) or ROPE_DT_F32
 *              (an extension for float32 attention); UNDEFINED -> ROPE_ERR_DTYPE.
 *   sin_out, cos_out  DEVICE [ntokens, head_size] of out_dtype, row-major, contiguous.
 * Errors: NULL, SHAPE (sum(seq_lens) != ntokens, seq_len <= 0), LIMIT, DTYPE,
 * UNSUPPORTED (alignment), HIP.  One kernel launch.
 */
rope_status rope_tables(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens,
                        int32_t batch, int32_t ntokens, int32_t head_size, float pos_scale,
                        rope_dtype out_dtype, void* sin_out, void* cos_out, void* hip_stream);

/*
 * rope_tables_ex — rope_tables with a pairing (table column layout) and an angle mode.
 * rope_tables(...) is rope_tables_ex(..., ROPE_PAIR_HALF, ROPE_ANGLE_F32, ...).  All other
 * arguments, limits and errors as for rope_tables; pairing or angle_mode out of range ->
 * ROPE_ERR_UNSUPPORTED.  One kernel launch.
 */
rope_status rope_tables_ex(const int32_t* pos, const float* inv_freq, const int32_t* seq_lens,
                           int32_t batch, int32_t ntokens, int32_t head_size, float pos_scale,
                           rope_dtype out_dtype, rope_pairing pairing, rope_angle_mode angle_mode,
                           void* sin_out, void* cos_out, void* hip_stream);

/*
 * Parameters of rope_qk and rope_flash_attn_fwd.
 *
 * Q has hq heads, K and V have hkv heads; hq % hkv == 0 and q head h reads kv head
 * h / (hq / hkv) (contiguous groups; [RoPE/GQA tutorial], sections 十一-十二: query
 * heads split into groups, each group sharing one K/V head).
 *
 * Token addressing.  Dense batches (cu_seqlens == NULL): sequence b, token s < seqlen of
 * head h lives at base + b*stride[0] + s*stride[1] + h*stride[2] + d*stride[3].  This
 * covers BNSD ([B, H, S, D], the input_layout of the [RoPE-fusion blog], section 三) and
 * BSND.  Packed varlen batches (cu_seqlens != NULL): token s of sequence b is packed row
 * t = cu_seqlens[b] + s at base + t*stride[1] + h*stride[2] + d*stride[3]; stride[0] is
 * ignored.  stride[3] (the head_dim stride) must be 1.  Strides are in elements.  The
 * attention calls (forward and backward) return ROPE_ERR_LIMIT when a K or V token stride
 * (stride[1]) is 2^26 bytes or more: the fused kernel addresses its key tiles with 32-bit
 * per-lane offsets.
 *
 * Tables (cos, sin) are [rows, head_dim] of table_dtype, row-major and contiguous, as
 * rope_tables writes them.  Row of token (b, s):
 *   varlen: the packed row cu_seqlens[b] + s;
 *   dense:  s when table_seq_rows == 0 (one table shared by every sequence), else
 *           b * table_seq_rows + s (table_seq_rows >= seqlen).
 * cos == sin == NULL disables the rotation (plain attention; rope_flash_attn_fwd only).
 *
 * Tables formed in the kernel: with cos == sin == NULL and pos != NULL the kernels compute
 * each table value they use from pos (int32, one per table row, rows indexed exactly as
 * the table rows above) and inv_freq ([inv_freq_rows, head_dim/2] float; row b serves
 * sequence b, or row 0 serves all when inv_freq_rows == 1), in ROPE_ANGLE_F32 mode, and
 * round it to dtype: the results equal those of the same call with the tables that
 * rope_tables_ex(pos, inv_freq, ..., pos_scale, dtype, pairing, ROPE_ANGLE_F32) writes
 * (the table computation of the [RoPE-fusion blog], section 5.1, done inside the fused
 * operator).  table_dtype and table_seq_rows keep their meaning for the row indexing.
 */
typedef struct rope_attn_params {
    uint32_t struct_size;       /* = sizeof(rope_attn_params), else ROPE_ERR_ABI */
    rope_dtype dtype;           /* q, k, v, out, out_q, out_k: F32 | F16 | BF16 */
    const void* q;              /* DEVICE, hq heads */
    const void* k;              /* DEVICE, hkv heads */
    const void* v;              /* DEVICE, hkv heads (rope_flash_attn_fwd only) */
    void* out;                  /* DEVICE, hq heads, layout by o_stride (rope_flash_attn_fwd) */
    void* out_q;                /* DEVICE, rope_qk only: rotated q, strides q_stride; may equal q */
    void* out_k;                /* DEVICE, rope_qk only: rotated k, strides k_stride; may equal k */
    float* lse;                 /* DEVICE float [hq, ntokens] or NULL: natural-log sum of exp of the
                                   scaled scores per query row (token index as for tables, varlen:
                                   packed row, dense: b*seqlen + s) */
    int32_t batch;              /* number of sequences, >= 1 */
    int32_t hq, hkv;            /* heads of q and of k/v */
    int32_t head_dim;           /* rope_qk: multiple of 32, <= 2048; attention: 64 or 128 */
    int32_t seqlen;             /* dense: tokens per sequence; varlen: ignored (set 0) */
    int32_t max_seqlen;         /* varlen: HOST upper bound of every sequence length */
    int32_t ntokens;            /* varlen: HOST total tokens = cu_seqlens[batch]; dense: 0 or batch*seqlen */
    int32_t causal;             /* 0 or 1 (rope_flash_attn_fwd) */
    const int32_t* cu_seqlens;  /* DEVICE [batch + 1] int32 prefix sums starting at 0, or NULL = dense */
    int64_t q_stride[4];        /* {batch, token, head, dim} in elements */
    int64_t k_stride[4];
    int64_t v_stride[4];
    int64_t o_stride[4];
    const void* cos;            /* DEVICE [rows, head_dim] of table_dtype, or NULL (with sin) */
    const void* sin;
    rope_dtype table_dtype;     /* must equal dtype when tables are given */
    int32_t table_seq_rows;     /* dense only, see above */
    float softmax_scale;        /* multiplies q.k before the softmax; the caller passes 1/sqrt(head_dim)
                                   ([FlashAttention blog]: Softmax(QK^T/sqrt(d))V) */
    rope_pairing pairing;       /* pair layout of the rotation and of the tables */
    const int32_t* pos;         /* DEVICE int32 [table rows] or NULL: positions for tables formed in
                                   the kernel (used only when cos == sin == NULL) */
    const float* inv_freq;      /* DEVICE float [inv_freq_rows, head_dim/2] (with pos) */
    int32_t inv_freq_rows;      /* 1 or batch (with pos) */
    float pos_scale;            /* linear position scaling, finite and > 0 (with pos) */
    uint8_t rsv[16];            /* reserved, must be zero (cf. the rsv[] of DynamicNTKParam) */
} rope_attn_params;

/*
 * rope_qk — standalone RoPE of Q and K: the Rope op that consumes the DynamicNTK
 * tables ([DynamicNTKOperation], 算子上下文: q, k, sin, cos in, rotated q, k out),
 * the unfused "RoPE, write to HBM, then attention" step of the [RoPE-fusion blog],
 * section 二.  For every token and head of q and of k, with x a head row of length
 * D = head_dim and the token's table rows cos, sin:
 *   x'[j] = x[j]*cos[j] + rotate_half(x)[j]*sin[j],  rotate_half(x) = cat(-x[D/2:], x[:D/2])
 * (ROPE_PAIR_HALF; with ROPE_PAIR_INTERLEAVED the partner of x[2i] is x[2i+1] instead),
 * computed in float32 and rounded to nearest-even into dtype.  All D table columns are
 * read (or formed in the kernel from pos and inv_freq, see above).  Uses q, k, out_q, out_k, cos, sin, table_dtype, table_seq_rows, batch, hq, hkv,
 * head_dim, seqlen / cu_seqlens / ntokens, q_stride (also for out_q), k_stride (also for
 * out_k).  In-place (out_q == q, out_k == k) is allowed; other overlap is not.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, HIP.  One kernel launch.
 */
rope_status rope_qk(const rope_attn_params* p, void* hip_stream);

/*
 * rope_flash_attn_fwd — RoPE fused into a FlashAttention forward pass
 * ([RoPE-fusion blog], section 三: one fused operator so rotated Q/K never return to
 * HBM; [FlashAttention blog]: tiled QK^T, online softmax with a running row max and
 * row sum, then PV).  For every sequence b, q head h and query s of that sequence:
 *   q' = rope(q[b, s, h]),  k'_j = rope(k[b, j, h / g])   (the rope_qk formula)
 *   out[b, s, h] = sum_j softmax_j(softmax_scale * q'.k'_j) v[b, j, h / g]
 * over keys j <= s when causal (within the sequence), else all j < length.
 * With ROPE_PAIR_HALF the kernel reads only table columns [0, head_dim/2) and applies them
 * to both halves: tables must be in the cat(freq, freq) form that rope_tables produces
 * (unchecked).  With ROPE_PAIR_INTERLEAVED all columns are read.  Tables may instead be
 * formed in the kernel from pos and inv_freq (see the parameters).
 * Supported: head_dim 64 or 128 with F16, BF16 (fp16/bf16 matrix cores with float32
 * accumulation); head_dim 64 with F32 (float32 matrix cores).  Optional lse output (see above).
 * Varlen lengths live on the device and are not validated; the kernels clamp them instead
 * ([DynamicNTKOperation], 约束说明, requires positive lengths that sum to ntokens): sequence b
 * covers the packed rows [s_b, s_b + L_b) with s_b = min(max(cu_seqlens[b], 0), ntokens) and
 * L_b = max(0, min(cu_seqlens[b + 1] - s_b, max_seqlen, ntokens - s_b)), and is computed as a
 * sequence of L_b tokens.  No access leaves the packed rows; rows of out and lse outside
 * every such range are left unwritten.  With well-formed cu_seqlens nothing is clamped.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, HIP.  One kernel launch.
 */
rope_status rope_flash_attn_fwd(const rope_attn_params* p, void* hip_stream);

/*
 * rope_flash_attn_fwd_ws — the same operation and result as rope_flash_attn_fwd (bit for bit),
 * with a caller-owned workspace that lets the library rotate each key once instead of in
 * every workgroup that stages it.  The fused kernel of [RoPE-fusion blog], section 三,
 * rotates a K tile wherever it is staged; a kv head's key is staged by every query tile and
 * head group that reaches it, so on long sequences the repeated rotation costs more than
 * one HBM round trip of k' (hkv heads: under GQA a fraction of q's bytes), which this call
 * accepts while q' still never reaches HBM.  When rope_flash_attn_fwd_workspace_size(p) > 0
 * the call runs two launches on hip_stream: a pre-pass that writes k' = rope(k) of every
 * key row and kv head (the rope_qk formula and rounding, reading only table columns
 * [0, head_dim/2) with ROPE_PAIR_HALF, as the fused kernel does) into the workspace, then
 * the fused kernel with q rotated in registers as before and the k' tiles staged as they
 * are; rotated q never leaves the registers.  When the size is 0 (no rotation, F32, short
 * sequences where in-loop rotation is cheaper, or varlen with tables formed from
 * per-sequence inverse frequencies) it is rope_flash_attn_fwd and the workspace is unused.
 * workspace: DEVICE, 256-byte aligned, >= the size, not overlapping any input or output;
 * after the call it holds k' of dtype as [batch, hkv, seqlen, head_dim] (dense) or
 * [hkv, ntokens, head_dim] (varlen) and is only used by this call's kernels (reuse it once
 * the stream has passed them).  Errors: those of rope_flash_attn_fwd, and ROPE_ERR_WORKSPACE when the size
 * is > 0 and the workspace is NULL, misaligned or smaller.
 */
rope_status rope_flash_attn_fwd_ws(const rope_attn_params* p, void* workspace, uint64_t workspace_bytes,
                                   void* hip_stream);

/* Workspace bytes rope_flash_attn_fwd_ws uses for these parameters (0: none, in-loop
 * rotation), or 0 when the parameters are invalid.  Host only. */
uint64_t rope_flash_attn_fwd_workspace_size(const rope_attn_params* p);

/*
 * Parameters of rope_flash_attn_bwd: the forward call's parameters plus the gradients.
 *
 * fwd.out must hold the forward output O and fwd.lse its lse (both from the forward call
 * with the same inputs; lse is required here).  Rotation: tables (fwd.cos, fwd.sin, with
 * fwd.pairing) or none (both NULL); tables formed in the kernel (fwd.pos) are not served
 * by the backward (ROPE_ERR_UNSUPPORTED).  dout, dq have hq heads, dk, dv hkv heads; strides
 * {batch, token, head, dim} as for the forward tensors (dim stride 1).  dq, dk, dv are
 * written in full (every element of every valid token) and must not overlap the inputs.
 */
typedef struct rope_attn_bwd_params {
    uint32_t struct_size;       /* = sizeof(rope_attn_bwd_params), else ROPE_ERR_ABI */
    rope_attn_params fwd;       /* the forward parameters (fwd.struct_size checked too) */
    const void* dout;           /* DEVICE gradient of the output, like fwd.out */
    void* dq;                   /* DEVICE, like q */
    void* dk;                   /* DEVICE, like k */
    void* dv;                   /* DEVICE, like v */
    int64_t do_stride[4];       /* {batch, token, head, dim} in elements */
    int64_t dq_stride[4];
    int64_t dk_stride[4];
    int64_t dv_stride[4];
    void* workspace;            /* DEVICE scratch, 256-byte aligned, >= rope_flash_attn_bwd_workspace_size() */
    uint64_t workspace_bytes;
    uint8_t rsv[16];            /* reserved, must be zero */
} rope_attn_bwd_params;

/* Workspace bytes rope_flash_attn_bwd needs, or 0 when the shapes are invalid: one float
 * per query row and q head (rowsum(dO * O)), then the rotated rows q' (rows x hq x head_dim)
 * and k' (rows x hkv x head_dim) in the dtype, each part 256-byte aligned.  Host only. */
uint64_t rope_flash_attn_bwd_workspace_size(const rope_attn_bwd_params* p);

/*
 * rope_flash_attn_bwd — gradients of rope_flash_attn_fwd: with the forward's
 * O = softmax(s * q'k'^T) V per (sequence, q head) (s = softmax_scale, q' and k' the rotated
 * rows), and dO the gradient of O,
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dq' = s * dS k',  dk' = s * dS^T q',  dq = M^T dq',  dk = M^T dk'
 * with M each token's Rope-op matrix (its transpose undoes the rotation), and the dk, dv of
 * a kv head summed over the q heads of its group ([RoPE/GQA tutorial], sections 十一-十二).
 * The [FlashAttention blog] states that the operator serves training; the gradients are
 * those of the forward definition.  P is recomputed from the forward's lse, never stored.
 * Supported: F16/BF16, head_dim 64 or 128, causal or not, dense or varlen, GQA, both
 * pairings.  float32 accumulation; outputs rounded once to dtype.  Varlen lengths are
 * clamped exactly as in rope_flash_attn_fwd; rows of dq, dk, dv outside every clamped
 * sequence are left unwritten.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, WORKSPACE, HIP.  Three kernel launches
 * (row deltas with the rotated q', k'; dk/dv; dq).
 */
rope_status rope_flash_attn_bwd(const rope_attn_bwd_params* p, void* hip_stream);

/* sizeof(rope_attn_bwd_params) as compiled into the library (for bindings to check). */
uint32_t rope_attn_bwd_params_size(void);

/*
 * Parameters of rope_kv_rms_norm_rope_cache.
 *
 * New tokens are rows t < ntokens of k and v: head h of token t lives at
 * base + t*stride[0] + h*stride[1] + d (strides {token, head} in elements, dim stride 1).
 *
 * Cache addressing.  A cache slot s is split into block s / block_size and offset
 * s % block_size; head h of slot s lives at
 *   cache + (s / block_size)*c_stride[0] + (s % block_size)*c_stride[1] + h*c_stride[2] + d.
 * block_size = the cache length of one sequence gives a contiguous per-sequence cache,
 * [B, S_max, hkv, D] (c_stride {S_max*hkv*D, hkv*D, D}) or [B, hkv, S_max, D]
 * (c_stride {hkv*S_max*D, D, S_max*D}); a smaller block_size gives a paged cache
 * [num_blocks, block_size, hkv, D] (the paged KV-cache management the [FlashAttention
 * blog] points to in its KV-cache pitfall).
 */
typedef struct rope_kv_cache_params {
    uint32_t struct_size;       /* = sizeof(rope_kv_cache_params), else ROPE_ERR_ABI */
    rope_dtype dtype;           /* k, v, cos, sin, k_cache, v_cache: F32 | F16 | BF16 */
    const void* k;              /* DEVICE [ntokens, hkv, head_dim] by k_stride */
    const void* v;              /* DEVICE [ntokens, hkv, head_dim] by v_stride; NULL together with
                                   v_cache = K only.  k, v, cos, sin and slots may be NULL when
                                   ntokens == 0 */
    const float* gamma;         /* DEVICE float [head_dim] RMSNorm weight; NULL = no normalisation */
    const void* cos;            /* DEVICE [ntokens, head_dim] of dtype: row t serves new token t */
    const void* sin;
    const int64_t* slots;       /* DEVICE int64 [ntokens]: cache slot of each new token; a slot < 0 or
                                   >= num_blocks * block_size skips the token (nothing written) */
    void* k_cache;              /* DEVICE, addressed by kc_stride as above */
    void* v_cache;              /* DEVICE, addressed by vc_stride; NULL together with v */
    int32_t ntokens;            /* new tokens, >= 0 (0: nothing is enqueued) */
    int32_t hkv;                /* heads of k and v, >= 1 */
    int32_t head_dim;           /* multiple of 32, <= ROPE_MAX_HEAD_SIZE */
    int32_t block_size;         /* slots per cache block, >= 1 */
    int32_t num_blocks;         /* cache blocks, >= 1 */
    float eps;                  /* RMSNorm epsilon, finite and >= 0 */
    int64_t k_stride[2];        /* {token, head} in elements */
    int64_t v_stride[2];
    int64_t kc_stride[3];       /* {block, offset in block, head} in elements */
    int64_t vc_stride[3];
    rope_pairing pairing;       /* pair layout of the rotation and of the tables */
    uint8_t rsv[12];            /* reserved, must be zero */
} rope_kv_cache_params;

/*
 * rope_kv_rms_norm_rope_cache — the fused "RMSNorm, RoPE, write to the KV cache" step
 * that precedes attention (kv_rms_norm_rope_cache, named in the [RoPE-fusion blog],
 * section 五; the pages do not define it, this is the reading taken).  For every new
 * token t with a valid slot s = slots[t] and every kv head h, with x = k[t, h] (length
 * D = head_dim):
 *   y = gamma * x / sqrt(mean(x^2) + eps)           ([RoPE/GQA tutorial], section 八;
 *                                                     y = x when gamma == NULL)
 *   k_cache[s, h] = y*cos[t] + rotate_half(y)*sin[t]  (the rope_qk formula, all D columns)
 *   v_cache[s, h] = v[t, h]                           (bit-exact copy)
 * computed in float32 and rounded once to nearest-even into dtype.  Two tokens with the
 * same slot race (which one lands is unspecified).  k and v must not overlap the caches.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, HIP.  One kernel launch (none
 * when ntokens == 0).
 */
rope_status rope_kv_rms_norm_rope_cache(const rope_kv_cache_params* p, void* hip_stream);

/* sizeof(rope_kv_cache_params) as compiled into the library (for bindings to check). */
uint32_t rope_kv_cache_params_size(void);

/*
 * Parameters of rope_decode_attn_fwd: one decode step over a (paged) KV cache.
 *
 * Sequence b has cache_seqlens[b] tokens in the cache (the new token included, its K' and
 * V already written, e.g. by rope_kv_rms_norm_rope_cache).  Its token j lives in logical
 * block j / block_size at offset j % block_size; the physical block is
 * block_table[b * max_blocks_per_seq + j / block_size], or b * max_blocks_per_seq +
 * j / block_size when block_table is NULL (a contiguous per-sequence cache).  Head h of a
 * physical slot is addressed as in rope_kv_cache_params (kc_stride, vc_stride).
 */
typedef struct rope_decode_params {
    uint32_t struct_size;         /* = sizeof(rope_decode_params), else ROPE_ERR_ABI */
    rope_dtype dtype;             /* q, cos, sin, k_cache, v_cache, out: F16 | BF16 */
    const void* q;                /* DEVICE [batch, hq, head_dim] by q_stride: the new queries, not rotated */
    const void* cos;              /* DEVICE [batch, head_dim] of dtype: row b rotates sequence b's query
                                     (the table row of its position); NULL with sin = no rotation */
    const void* sin;
    const void* k_cache;          /* DEVICE, keys as stored (already rotated) */
    const void* v_cache;          /* DEVICE */
    const int32_t* block_table;   /* DEVICE int32 [batch, max_blocks_per_seq], or NULL (see above) */
    const int32_t* cache_seqlens; /* DEVICE int32 [batch]: cached tokens per sequence */
    void* out;                    /* DEVICE [batch, hq, head_dim] by o_stride */
    float* lse;                   /* DEVICE float [batch, hq] natural-log sum of exp of the scaled
                                     scores, or NULL */
    void* workspace;              /* DEVICE scratch, 256-byte aligned, >= rope_decode_workspace_size() */
    uint64_t workspace_bytes;     /* size of workspace in bytes */
    int32_t batch;                /* sequences, 1..65535 */
    int32_t hq, hkv;              /* query heads and cached kv heads, hq % hkv == 0 */
    int32_t head_dim;             /* 64 or 128 */
    int32_t block_size;           /* cache slots per block, >= 1 */
    int32_t max_blocks_per_seq;   /* block-table row length, >= 1 */
    int32_t num_blocks;           /* physical cache blocks, >= 1 */
    int32_t max_seqlen;           /* HOST bound of cache_seqlens, 1..max_blocks_per_seq*block_size */
    int32_t num_splits;           /* key-range splits per sequence: 0 = the library's choice, else 1..256;
                                     each split covers the same number of keys, ceil(max_seqlen /
                                     num_splits) rounded up to 32, so shorter sequences leave their last
                                     splits empty */
    float softmax_scale;          /* multiplies q.k before the softmax */
    int64_t q_stride[2];          /* {batch, head} in elements; head_dim stride 1 */
    int64_t o_stride[2];
    int64_t kc_stride[3];         /* {block, offset in block, head} in elements */
    int64_t vc_stride[3];
    rope_pairing pairing;         /* pair layout of the query rotation and of its tables */
    uint8_t rsv[12];              /* reserved, must be zero */
} rope_decode_params;

/*
 * rope_decode_workspace_size — bytes of workspace rope_decode_attn_fwd needs for these
 * parameters (batch, hq, head_dim, hkv, max_seqlen, num_splits are read), or 0 when they
 * are invalid.  Host only.
 */
uint64_t rope_decode_workspace_size(const rope_decode_params* p);

/*
 * rope_decode_attn_fwd — decode-step RoPE + GQA attention over a KV cache (the step after
 * prefill whose memory traffic GQA exists to cut: [RoPE/GQA tutorial], sections 十一-十二,
 * the KV cache shrinks by Hq/Hkv; the paged cache of the [FlashAttention blog]'s KV-cache
 * pitfall).  For every sequence b and q head h, with g = hq / hkv and L = cache_seqlens[b]:
 *   q' = rope(q[b, h]) with the table row b (the rope_qk formula; no rotation when cos and
 *        sin are NULL)
 *   out[b, h] = sum_{j < L} softmax_j(softmax_scale * q'.K[b, j, h / g]) V[b, j, h / g]
 * with K, V read from the cache as stored.  Every kv head's cache is read once for its g
 * query heads.  The key range of each sequence is split over num_splits partial passes
 * that a second kernel merges (both on hip_stream; the workspace holds the partial
 * results and must not be shared by calls that overlap).  Device-side values are trusted
 * as follows: a length above max_seqlen is clamped to it; a length <= 0 gives a zero
 * output and lse = -inf; block-table entries must lie in [0, num_blocks) (others are
 * clamped into range, so the cache is never read out of bounds, but the result is then
 * meaningless).  float32 accumulation; the output is rounded once to dtype.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, WORKSPACE, HIP.  Two kernel launches.
 */
rope_status rope_decode_attn_fwd(const rope_decode_params* p, void* hip_stream);

/* sizeof(rope_decode_params) as compiled into the library (for bindings to check). */
uint32_t rope_decode_params_size(void);

/* Largest scratch rope_decode_attn_fwd_noalloc can use: 16 MiB per GPU. */
#define ROPE_DECODE_NOALLOC_MAX_BYTES ((uint64_t)16 << 20)

/*
 * rope_decode_attn_fwd_noalloc — rope_decode_attn_fwd for callers that cannot allocate
 * device memory or set up a workspace per call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same computation, same kernels and the same
 * result bit for bit; p->workspace and p->workspace_bytes are ignored.  The split partials
 * go to a scratch array of ROPE_DECODE_NOALLOC_MAX_BYTES that the library holds on every GPU
 * it runs on until the process ends; a call whose rope_decode_workspace_size exceeds it
 * returns ROPE_ERR_LIMIT (fewer num_splits reduce the need).  The entry point allocates
 * nothing: the scratch address is looked up (hipGetSymbolAddress) on the first call on each
 * device.  hip_stream must belong to the current device (else ROPE_ERR_HIP).  Every call on
 * one GPU shares that GPU's scratch: calls that overlap in time on one GPU (other streams,
 * other threads) race and must be serialised by the caller; calls in order on one stream
 * are safe.  Nothing in the scratch needs clearing between calls.
 * Errors: NULL, SHAPE, DTYPE, LIMIT, UNSUPPORTED, ABI, HIP.  Two kernel launches.
 */
rope_status rope_decode_attn_fwd_noalloc(const rope_decode_params* p, void* hip_stream);

/* Static text for a status code ("ROPE_OK", ...); never NULL. */
const char* rope_status_str(rope_status s);

/* ROPE_FA_ABI_VERSION of the loaded library. */
int32_t rope_abi_version(void);

/* sizeof(rope_attn_params) as compiled into the library (for bindings to check). */
uint32_t rope_attn_params_size(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_FA_H */
