/*
 * gmla.h -- C ABI of the MI355X (gfx950) library for causal softmax attention in
 * Gated MLA ("Multi-head Latent Attention") layers.
 *
 * What it computes (the pages that define it):
 *   - "Gated MLA" (ai-engineer-exhaustive.pages.dev, research/kimik3/k3-gated-mla),
 *     section "Start from familiar attention": per head, A = softmax(Q K^T / sqrt(D_h) + M),
 *     head context A V; C = X W_c^T; K = C W_k^T; V = C W_v^T.
 *     Section "The channel-wise output gate": Y = [sigmoid(X W_g^T) (.) O~] W_o^T.
 *     Section "Split attention into heads": head h owns channels h*D_h .. (h+1)*D_h - 1.
 *   - "Kimi K3 - Softmax over keys" (atlas.klimoza.dev): the softmax formula over a
 *     query's own and earlier keys, computed in float32; decode shape [B, 96, 1, 1001].
 *   - "Kimi K2 - Construct causal mask" (atlas.klimoza.dev): M[t,s] = 0 for s <= t,
 *     -inf for s > t; positions continue from the cached length.
 *   - "Le Transformer et l'attention" (mkdocs.reaper.mx, Kimi K3 fondations): 96 heads of
 *     width 128, latent width (kv_lora_rank) 512, no positional encoding in MLA layers.
 *
 * Conventions shared by every entry point:
 *   - Every tensor argument is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or retains device memory, and never writes an input.
 *   - dtype is GMLA_F32 (IEEE float) or GMLA_BF16 (bfloat16).  All tensors of one call
 *     share that dtype ("Gated MLA", section "Constraints").  Accumulation and the
 *     softmax are always float32; bf16 outputs are rounded to nearest even.
 *   - All arguments are validated on the host before any HIP call; a bad argument
 *     returns a negative status and launches nothing.
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls are
 *     asynchronous and stream-ordered; a launch failure returns GMLA_ERR_HIP.
 *   - Apart from the fixed scratch array of gmla_attend_decode_noalloc (see there), the
 *     library holds no mutable global state, so calls from several host threads are
 *     safe; calls whose outputs alias their inputs are not supported.
 *   - Sequence lengths (T, Tq, Tk, N) are at most 2^31 - 16385: the kernels index rows
 *     with 32-bit integers and may step one tile past the last row; longer sequences
 *     return GMLA_ERR_UNSUPPORTED.
 *   - Sizes are element counts; strides are element strides.
 */
#ifndef GMLA_H
#define GMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GMLA_F32 = 0, GMLA_BF16 = 1 } gmla_dtype;

typedef enum {
  GMLA_OK = 0,
  GMLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad flag, misaligned pointer */
  GMLA_ERR_UNSUPPORTED = -2, /* valid, but a shape/dtype the library has no kernel for */
  GMLA_ERR_WORKSPACE = -3,   /* decode workspace missing or too small */
  GMLA_ERR_HIP = -4,         /* the HIP runtime reported an error (no device, launch failure) */
  GMLA_ERR_TOO_LARGE = -5    /* the fixed scratch of a no-allocation call is too small */
} gmla_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* gmla_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int gmla_version(void);

/*
 * Causal (or full) attention of T queries against the same T keys, every head
 * independent; optional channel-wise sigmoid gate fused into the output.
 *
 * Computes, for batch b, token t, head h, channel d (0 <= d < D):
 *   O[b, t, h*D + d] = g * sum_{s visible} A[t,s] V[b, s, h, d],
 *   A[t,s] = exp(S[t,s]) / sum_{u visible} exp(S[t,u]),
 *   S[t,s] = scale * sum_d Q[b,t,h,d] K[b,s,h,d],
 * where "visible" is s <= t when causal = 1 ("Kimi K2 - Construct causal mask") and
 * every s < T when causal = 0 ("Gated MLA", section "A small causal example",
 * non-causal mode), and g = 1 / (1 + exp(-G[b, t, h*D + d])) if G is given, else 1
 * ("Gated MLA", section "The channel-wise output gate").  No positional encoding.
 *
 *   Q, K, V : element (b, t, h, d) at b*strides[0] + t*strides[1] + h*strides[2] + d;
 *             strides == NULL means contiguous [B, T, H, D] (strides H*T*D, H*D, D).
 *   G       : nullable, contiguous [B, T, H*D] gate logits.
 *   O       : contiguous [B, T, H*D] output (heads joined back to model width).
 *   scale   : usually 1/sqrt(D) ("Gated MLA", the attention formula).
 * Supported: GMLA_BF16 with D = 128 (MFMA kernel) or D in {32, 64}; GMLA_F32 with
 * D in {32, 64, 128}.  Every pointer must be aligned to its element size.  For bf16
 * with D = 128: Q, K, V, G and O 16-byte aligned and every stride a multiple of 8
 * (else GMLA_ERR_INVALID_ARG), and the token stride below 2^24 elements (byte offsets
 * inside one 64-row key tile are 32-bit; else GMLA_ERR_UNSUPPORTED).
 */
int gmla_attend_prefill(int dtype, int B, int T, int H, int D, float scale, int causal,
                        const void* Q, const void* K, const void* V, const int64_t* strides,
                        const void* G, void* O, void* stream);

/*
 * Attention of a chunk of Tq queries that follow Tk - Tq cached tokens (chunked
 * prefill, several new tokens at once): query i of the chunk sits at absolute
 * position p_i = i + Tk - Tq, positions continuing from the cached length ("Kimi K2 -
 * Construct causal mask"; "Kimi K3 - Softmax over keys", decode at position 1000 with
 * 1001 keys), and with causal = 1 it sees the keys s <= p_i (bottom-right aligned);
 * with causal = 0 it sees all Tk keys.  Same formula, gate and supported types as
 * gmla_attend_prefill, which is this call with Tq = Tk and one set of strides.
 *
 *   Q : element (b, i, h, d) at b*q_strides[0] + i*q_strides[1] + h*q_strides[2] + d
 *       (NULL: contiguous [B, Tq, H, D]).
 *   K,V: element (b, s, h, d) at b*kv_strides[0] + s*kv_strides[1] + h*kv_strides[2] + d
 *       (NULL: contiguous [B, Tk, H, D]), s < Tk: the cache followed by the chunk.
 *   G : nullable, contiguous [B, Tq, H*D];  O : contiguous [B, Tq, H*D].
 * Requires 1 <= Tq <= Tk (else GMLA_ERR_INVALID_ARG).  Alignment, stride and length
 * limits as for gmla_attend_prefill (the key token stride is kv_strides[1]).
 */
int gmla_attend_chunk(int dtype, int B, int Tq, int Tk, int H, int D, float scale, int causal,
                      const void* Q, const int64_t* q_strides, const void* K, const void* V,
                      const int64_t* kv_strides, const void* G, void* O, void* stream);

/*
 * Causal (or full) prefill whose keys and values are rebuilt from the latent rows when
 * attention runs ("Gated MLA", section "Start from familiar attention": C is the cached
 * latent, K = C W_k^T and V = C W_v^T): the same result as gmla_latent_expand followed by
 * gmla_attend_prefill, in one persistent launch.  Expansion tasks compute the keys and
 * values of (batch, head, 128 latent rows) once each, into the workspace; attention tasks
 * (query blocks of 128, heaviest first) start as soon as the rows they read are ready.
 *
 *   Q : element (b, t, h, d) at b*q_strides[0] + t*q_strides[1] + h*q_strides[2] + d
 *       (NULL: contiguous [B, T, H, D]).
 *   C : contiguous [B, T, d_c] latent rows.  W_k, W_v : contiguous [H*D, d_c].
 *   G : nullable, contiguous [B, T, H*D] gate logits.  O : contiguous [B, T, H*D].
 *   workspace: at least gmla_prefill_latent_workspace_bytes(B, T, H, D) bytes, 256-byte
 *       aligned, owned by the caller (the keys and values, plus ready flags that the
 *       call clears itself), not shared with a concurrent call (else GMLA_ERR_WORKSPACE).
 * Supported: GMLA_BF16, D = 128, d_c a multiple of 32 (else GMLA_ERR_UNSUPPORTED); Q, C,
 * W_k, W_v, G, O 16-byte aligned and Q's strides multiples of 8 (else
 * GMLA_ERR_INVALID_ARG).  The tasks are queued per accelerator die, so the device must
 * expose all eight dies of the MI355X (a single partition, 256 compute units; else
 * GMLA_ERR_UNSUPPORTED).  Launches a small clearing kernel, then the fused kernel.
 */
size_t gmla_prefill_latent_workspace_bytes(int B, int T, int H, int D);
int gmla_attend_prefill_latent(int dtype, int B, int T, int H, int D, int d_c, float scale,
                               int causal, const void* Q, const int64_t* q_strides, const void* C,
                               const void* W_k, const void* W_v, const void* G, void* O,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention over a packed batch of sequences of different lengths (ragged prefill or
 * chunked prefill with a different cached length per sequence).  Sequence b owns the
 * query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 (Tq_b of them) and the key/value
 * rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1 (Tk_b); its query i sits at position
 * i + Tk_b - Tq_b, positions continuing from that sequence's cached length ("Kimi K2 -
 * Construct causal mask"), and with causal = 1 sees its keys s <= i + Tk_b - Tq_b
 * (bottom-right aligned per sequence); with causal = 0 all Tk_b of them.  Same formula
 * and gate as gmla_attend_prefill.  A query that sees no key (only possible when
 * Tq_b > Tk_b) gets an all-zero output row.
 *
 *   Q    : row r, head h at r*q_strides[0] + h*q_strides[1] (NULL: contiguous
 *          [total_q, H, D]);  K, V: likewise with kv_strides ([total_k, H, D]).
 *   cu_seqlens_q, cu_seqlens_k : DEVICE arrays of B + 1 int32 row offsets,
 *          non-decreasing; every Tq_b <= max_seqlen_q (rows past it are not computed)
 *          and every Tk_b <= 2^31 - 16385.  The offsets are read by the kernels only, so
 *          the caller guarantees they address rows inside Q, K, V, G and O.
 *   G    : nullable, contiguous [total_q, H*D];  O : contiguous [total_q, H*D].
 * Supported types, alignment and stride limits as for gmla_attend_prefill.
 */
int gmla_attend_varlen(int dtype, int B, int H, int D, float scale, int causal, const void* Q,
                       const int64_t* q_strides, const int* cu_seqlens_q, int max_seqlen_q,
                       const void* K, const void* V, const int64_t* kv_strides,
                       const int* cu_seqlens_k, int max_seqlen_k, const void* G, void* O,
                       void* stream);

/*
 * Decode: one new query per (b, h) against N cached keys.  The query sits at
 * position N - 1, so every cached key is visible ("Kimi K3 - Softmax over keys":
 * the query at p = 1000 reads 1001 keys).  The keys are split into num_splits
 * ranges, each reduced to a running maximum, sum and weighted value sum in float32,
 * and the ranges are merged by log-sum-exp; the result equals the single softmax
 * over all N keys up to rounding.
 *
 *   Q  : contiguous [B, H, D].
 *   K,V: element (b, h, n, d) at b*kv_strides[0] + h*kv_strides[1] + n*kv_strides[2] + d;
 *        kv_strides == NULL means contiguous [B, H, N, D].
 *   G  : nullable, contiguous [B, H*D] gate logits; O: contiguous [B, H*D].
 *   workspace: device scratch of at least gmla_decode_workspace_bytes(B, H, N, D,
 *        num_splits) bytes (may be NULL when that is 0), owned by the caller, and not
 *        shared with a concurrent call.
 *   num_splits: 0 chooses automatically (gmla_decode_num_splits); at most 4096.
 * Supported: D = 128 (bf16 or f32), or D in {32, 64} (f32 or bf16).  Q, K and V must be
 * 16-byte aligned and every kv_stride times the element size a multiple of 16 bytes
 * (rows are read 16 bytes at a time, float32 too); O and G aligned to their element
 * size.  Else GMLA_ERR_INVALID_ARG.
 */
int gmla_decode_num_splits(int B, int H, int N, int D);
size_t gmla_decode_workspace_bytes(int B, int H, int N, int D, int num_splits);
int gmla_attend_decode(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                       const void* K, const void* V, const int64_t* kv_strides, const void* G,
                       void* O, void* workspace, size_t workspace_bytes, int num_splits,
                       void* stream);

/*
 * gmla_attend_decode with a cache length per batch row: row b holds kv_lens[b] keys
 * (a DEVICE array of B int32; values are clamped to [0, N], N being the cache capacity
 * that kv_strides describe), and its query sits at position kv_lens[b] - 1, seeing all
 * of them ("Kimi K2 - Construct causal mask": positions continue from the cached
 * length).  A row with no key gets an all-zero output.  Workspace, splits (taken over
 * the capacity N), types and limits as for gmla_attend_decode.
 */
int gmla_attend_decode_varlen(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                              const void* K, const void* V, const int64_t* kv_strides,
                              const int* kv_lens, const void* G, void* O, void* workspace,
                              size_t workspace_bytes, int num_splits, void* stream);

/*
 * Decode over the latent cache: one new query per (b, h) at position N - 1 against N
 * cached tokens that are stored only as latent rows c_n of width d_c ("Gated MLA",
 * section "Start from familiar attention": K = C W_k^T, V = C W_v^T; section "Common
 * mistakes to avoid": the cache is the compact latent tensor C; "Le Transformer et
 * l'attention", "MLA - compresser en un vecteur latent": 512 values per token).
 *
 * Computes, with W_k,h and W_v,h the rows h*D .. h*D + D - 1 of W_k and W_v:
 *   k_{h,n} = W_k,h c_n,  v_{h,n} = W_v,h c_n,
 *   O[b, h*D + d] = g * sum_n softmax_n(scale * q_{b,h} . k_{h,n}) v_{h,n}[d],
 * with the optional gate g = sigmoid(G[b, h*D + d]).  The keys and values are never
 * formed: the library uses the exact regrouping q'_{b,h} = scale W_k,h^T q_{b,h}
 * (scores q' . c_n) and o = W_v,h (sum_n p_n c_n), so each step reads the d_c latent
 * values per token (shared by all heads) and W_k, W_v once.
 *
 *   Q   : contiguous [B, H, D].
 *   C   : latent row (b, n) at b*c_strides[0] + n*c_strides[1], d_c contiguous values
 *         (NULL strides: contiguous [B, N, d_c]).
 *   W_k, W_v : contiguous [H*D, d_c] (stored [out, in]).
 *   G   : nullable, contiguous [B, H*D] gate logits;  O : contiguous [B, H*D].
 *   workspace: at least gmla_decode_latent_workspace_bytes(B, H, N, d_c, num_splits)
 *         bytes, 256-byte aligned, owned by the caller, not shared with a concurrent call
 *         (else GMLA_ERR_WORKSPACE).
 *   num_splits: key ranges per (b, 32-head block); 0 chooses (the ranges are rounded
 *         to multiples of 32 rows, so the count used can be smaller than asked).
 * Supported: GMLA_BF16, D = 128, d_c in {128, 256, 512} (else GMLA_ERR_UNSUPPORTED).
 * Q, C, W_k, W_v 16-byte aligned, C's strides multiples of 8 (else
 * GMLA_ERR_INVALID_ARG), c_strides[1] below 2^25, B and H at most 65535.
 */
int gmla_decode_latent_num_splits(int B, int H, int N, int d_c);
size_t gmla_decode_latent_workspace_bytes(int B, int H, int N, int d_c, int num_splits);
int gmla_attend_decode_latent(int dtype, int B, int H, int N, int D, int d_c, float scale,
                              const void* Q, const void* C, const int64_t* c_strides,
                              const void* W_k, const void* W_v, const void* G, void* O,
                              void* workspace, size_t workspace_bytes, int num_splits,
                              void* stream);

/*
 * gmla_attend_decode_latent with a cache length per batch row: row b holds kv_lens[b]
 * latent rows (a DEVICE array of B int32, 4-byte aligned; values are clamped to [0, N],
 * N being the capacity that c_strides describe), and its query sits at position
 * kv_lens[b] - 1, seeing all of them ("Kimi K2 - Construct causal mask": positions
 * continue from the cached length).  A row with no cached token gets an all-zero output.
 * Workspace, key ranges (planned over the capacity N), types and limits as for
 * gmla_attend_decode_latent; kv_lens NULL is GMLA_ERR_INVALID_ARG.
 */
int gmla_attend_decode_latent_varlen(int dtype, int B, int H, int N, int D, int d_c, float scale,
                                     const void* Q, const void* C, const int64_t* c_strides,
                                     const int* kv_lens, const void* W_k, const void* W_v,
                                     const void* G, void* O, void* workspace,
                                     size_t workspace_bytes, int num_splits, void* stream);

/*
 * gmla_attend_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops and harnesses that forbid
 * allocation).  Same arguments, results and limits as gmla_attend_decode, minus the
 * workspace: when a head is split, the partials go to a fixed scratch array of
 * gmla_decode_noalloc_scratch_bytes() bytes (4 MiB) that each GPU holds from its first
 * such call until the process ends.  A call whose split partials need more
 * (gmla_decode_workspace_bytes(B, H, N, D, splits) > that size) returns
 * GMLA_ERR_TOO_LARGE and launches nothing; the automatic split count never needs more
 * than about 2.2 MB for D = 128.  The call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  All such calls on one GPU share its array,
 * which keeps the last call's contents: calls that may overlap in time on one GPU (on
 * different streams, or from several host threads) race, so serialise them.
 */
size_t gmla_decode_noalloc_scratch_bytes(void);
int gmla_attend_decode_noalloc(int dtype, int B, int H, int N, int D, float scale,
                               const void* Q, const void* K, const void* V,
                               const int64_t* kv_strides, const void* G, void* O, int num_splits,
                               void* stream);

/*
 * Latent up-projection ("Gated MLA", section "Start from familiar attention":
 * K = C W_k^T, V = C W_v^T): C [M, d_c], W_k and W_v [d_model, d_c] (stored
 * [out, in]) -> K, V [M, d_model], all contiguous row-major.  One pass over C.
 */
int gmla_latent_expand(int dtype, int M, int d_c, int d_model, const void* C, const void* W_k,
                       const void* W_v, void* K, void* V, void* stream);

/*
 * Channel-wise sigmoid gate and output projection ("Gated MLA", section "The
 * channel-wise output gate"): Y = [sigmoid(G) (.) O~] W_o^T, the gate applied BEFORE
 * the projection.  O~ and G are [M, d_model]; W_o is [d_model, d_model] (stored
 * [out, in]); Y is [M, d_model].  G == NULL means O~ is already gated (for example
 * by gmla_attend_prefill); W_o == NULL means no projection (Y = gated O~).
 */
int gmla_gate_out(int dtype, int M, int d_model, const void* G, const void* O_tilde,
                  const void* W_o, void* Y, void* stream);

/*
 * gmla_gate_out with a caller workspace, for bf16 with both a gate and W_o: the gate is
 * applied by its own pass into the workspace (sigmoid(G) (.) O~ rounded to bf16, the same
 * operand gmla_gate_out forms while staging its GEMM tiles) and the projection then runs
 * on the LDS-pipelined GEMM.  At M = 2048, d_model = 12288 that is about 0.5 ms instead
 * of 2.0 ms.  gmla_gate_out_workspace_bytes(dtype, M, d_model) is the space it needs
 * (M * d_model * 2 bytes; 0 for fp32 and for d_model not a multiple of 64).  With no
 * gate, no W_o, fp32, or a NULL, misaligned (16 bytes) or smaller workspace the call is
 * exactly gmla_gate_out.  The workspace is owned by the caller, must not overlap G, O~,
 * W_o or Y (GMLA_ERR_INVALID_ARG) and is not shared with a concurrent call.  The result
 * equals gmla_gate_out's to the order of the float32 sums.
 */
size_t gmla_gate_out_workspace_bytes(int dtype, int M, int d_model);
int gmla_gate_out_ws(int dtype, int M, int d_model, const void* G, const void* O_tilde,
                     const void* W_o, void* Y, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Y [M, N] = X [M, K] W [N, K]^T, all contiguous row-major, float32 accumulation.
 * The projections of the layer: Q = X W_q^T, C = X W_c^T, G = X W_g^T ("Gated MLA",
 * sections "Start from familiar attention" and "The channel-wise output gate").
 */
int gmla_linear(int dtype, int M, int N, int K, const void* X, const void* W, void* Y,
                void* stream);

/*
 * gmla_linear with a caller workspace for products with few output tiles and a deep
 * reduction (the latent down-projection C = X W_c^T: 2048 x 512 x 12288): the reduction
 * is split into ranges computed in parallel into float partials in the workspace, then
 * summed and rounded to bf16 (a sum in another order than gmla_linear's, to float
 * rounding).  gmla_linear_workspace_bytes(M, N, K) is the space that path needs, 0 when
 * the shape does not use it; with a smaller or NULL workspace (or fp32) the call is
 * exactly gmla_linear.  The workspace (16-byte aligned) is owned by the caller and not
 * shared with a concurrent call.
 */
size_t gmla_linear_workspace_bytes(int M, int N, int K);
int gmla_linear_ws(int dtype, int M, int N, int K, const void* X, const void* W, void* Y,
                   void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMLA_H */
