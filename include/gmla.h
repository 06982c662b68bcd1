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
 *   - The library holds no mutable global state, so calls from several host threads
 *     are safe; calls whose outputs alias their inputs are not supported.
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
  GMLA_ERR_HIP = -4          /* the HIP runtime reported an error (no device, launch failure) */
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
 * D in {32, 64, 128}.  bf16 pointers must be 16-byte aligned, and strides multiples
 * of 8, for D = 128.
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
 * Requires 1 <= Tq <= Tk (else GMLA_ERR_INVALID_ARG).
 */
int gmla_attend_chunk(int dtype, int B, int Tq, int Tk, int H, int D, float scale, int causal,
                      const void* Q, const int64_t* q_strides, const void* K, const void* V,
                      const int64_t* kv_strides, const void* G, void* O, void* stream);

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
 *   num_splits: 0 chooses automatically (gmla_decode_num_splits).
 * Supported: D = 128 (bf16 or f32), or D in {32, 64} (f32 or bf16).
 */
int gmla_decode_num_splits(int B, int H, int N, int D);
size_t gmla_decode_workspace_bytes(int B, int H, int N, int D, int num_splits);
int gmla_attend_decode(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                       const void* K, const void* V, const int64_t* kv_strides, const void* G,
                       void* O, void* workspace, size_t workspace_bytes, int num_splits,
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
 * Y [M, N] = X [M, K] W [N, K]^T, all contiguous row-major, float32 accumulation.
 * The projections of the layer: Q = X W_q^T, C = X W_c^T, G = X W_g^T ("Gated MLA",
 * sections "Start from familiar attention" and "The channel-wise output gate").
 */
int gmla_linear(int dtype, int M, int N, int K, const void* X, const void* W, void* Y,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GMLA_H */
