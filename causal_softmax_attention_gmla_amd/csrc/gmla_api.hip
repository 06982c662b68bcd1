// C ABI of libgmla: argument validation on the host, kernel choice, launch.
// Every check runs before any HIP call, so a bad argument never touches the device.
#include "../../include/gmla.h"

#include <stdio.h>
#include <stdlib.h>

#include "gmla_internal.h"

using namespace gmla;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool valid_dtype(int dtype) { return dtype == GMLA_F32 || dtype == GMLA_BF16; }
size_t elem_size(int dtype) { return dtype == GMLA_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? GMLA_OK : GMLA_ERR_HIP; }

bool log_enabled() {
  static const bool on = [] {
    const char* v = getenv("GMLA_LOG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

}  // namespace

extern "C" {

const char* gmla_status_string(int status) {
  switch (status) {
    case GMLA_OK: return "GMLA_OK";
    case GMLA_ERR_INVALID_ARG: return "GMLA_ERR_INVALID_ARG";
    case GMLA_ERR_UNSUPPORTED: return "GMLA_ERR_UNSUPPORTED";
    case GMLA_ERR_WORKSPACE: return "GMLA_ERR_WORKSPACE";
    case GMLA_ERR_HIP: return "GMLA_ERR_HIP";
    default: return "GMLA_ERR_UNKNOWN";
  }
}

int gmla_version(void) { return kVersion; }

}  // extern "C"

namespace {

// Shared by the square prefill and the chunk entry points: Tq query rows against Tk >= Tq
// key rows, query i at position i + Tk - Tq.
int attend_impl(int dtype, int B, int Tq, int Tk, int H, int D, float scale, int causal,
                const void* Q, const int64_t* q_strides, const void* K, const void* V,
                const int64_t* kv_strides, const void* G, void* O, void* stream) {
  if (!valid_dtype(dtype) || B <= 0 || Tq <= 0 || Tk < Tq || H <= 0 || D <= 0)
    return GMLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GMLA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  PrefillArgs a;
  a.B = B; a.T = Tq; a.Tk = Tk; a.H = H; a.D = D;
  a.scale = scale;
  a.causal = causal;
  a.q = Q; a.k = K; a.v = V; a.g = G; a.o = O;
  if (q_strides) {
    a.qsb = q_strides[0]; a.qst = q_strides[1]; a.qsh = q_strides[2];
    if (a.qsb < 0 || a.qst < 0 || a.qsh < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.qsh = D;
    a.qst = (int64_t)H * D;
    a.qsb = (int64_t)Tq * H * D;
  }
  if (kv_strides) {
    a.sb = kv_strides[0]; a.st = kv_strides[1]; a.sh = kv_strides[2];
    if (a.sb < 0 || a.st < 0 || a.sh < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.sh = D;
    a.st = (int64_t)H * D;
    a.sb = (int64_t)Tk * H * D;
  }
  const size_t es = elem_size(dtype);
  if (!aligned(Q, es) || !aligned(K, es) || !aligned(V, es) || !aligned(O, es) ||
      (G && !aligned(G, es)))
    return GMLA_ERR_INVALID_ARG;
  if (D != 32 && D != 64 && D != 128) return GMLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == GMLA_BF16 && D == 128) {
    // 16-byte fragment loads: every row start must be 16-byte aligned
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        (G && !aligned(G, 16)) || a.sb % 8 || a.st % 8 || a.sh % 8 || a.qsb % 8 || a.qst % 8 ||
        a.qsh % 8)
      return GMLA_ERR_INVALID_ARG;
    // byte offsets inside one 64-token key tile are 32-bit
    if (a.st >= (int64_t)1 << 24) return GMLA_ERR_UNSUPPORTED;
    if (log_enabled())
      fprintf(stderr, "gmla: prefill bf16 mfma B=%d Tq=%d Tk=%d H=%d causal=%d gate=%d\n", B, Tq,
              Tk, H, causal, G != nullptr);
    e = launch_prefill_bf16_mfma(a, s);
  } else if (dtype == GMLA_BF16) {
    e = launch_prefill_simple_bf16(a, s);
  } else {
    e = launch_prefill_simple_f32(a, s);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

int gmla_attend_prefill(int dtype, int B, int T, int H, int D, float scale, int causal,
                        const void* Q, const void* K, const void* V, const int64_t* strides,
                        const void* G, void* O, void* stream) {
  return attend_impl(dtype, B, T, T, H, D, scale, causal, Q, strides, K, V, strides, G, O, stream);
}

int gmla_attend_chunk(int dtype, int B, int Tq, int Tk, int H, int D, float scale, int causal,
                      const void* Q, const int64_t* q_strides, const void* K, const void* V,
                      const int64_t* kv_strides, const void* G, void* O, void* stream) {
  return attend_impl(dtype, B, Tq, Tk, H, D, scale, causal, Q, q_strides, K, V, kv_strides, G, O,
                     stream);
}

int gmla_decode_num_splits(int B, int H, int N, int D) {
  (void)D;
  if (B <= 0 || H <= 0 || N <= 0) return 1;
  // Enough workgroups to cover the 256 compute units about eight times over, but
  // never a split shorter than 1024 keys: for short caches (one head = a few hundred
  // KB) the cross-split merge costs more than the extra parallelism gains.
  const long heads = (long)B * H;
  long splits = (2048 + heads - 1) / heads;
  long max_by_len = N / 1024;
  if (max_by_len < 1) max_by_len = 1;
  if (splits > max_by_len) splits = max_by_len;
  if (splits < 1) splits = 1;
  if (splits > 256) splits = 256;
  return (int)splits;
}

size_t gmla_decode_workspace_bytes(int B, int H, int N, int D, int num_splits) {
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return 0;
  if (num_splits == 0) num_splits = gmla_decode_num_splits(B, H, N, D);
  if (num_splits <= 1) return 0;
  return (size_t)B * H * num_splits * (D + 2) * sizeof(float);
}

int gmla_attend_decode(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                       const void* K, const void* V, const int64_t* kv_strides, const void* G,
                       void* O, void* workspace, size_t workspace_bytes, int num_splits,
                       void* stream) {
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 || D <= 0) return GMLA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 4096) return GMLA_ERR_INVALID_ARG;
  DecodeArgs a;
  a.B = B; a.H = H; a.N = N; a.D = D;
  a.scale = scale;
  a.q = Q; a.k = K; a.v = V; a.g = G; a.o = O;
  if (kv_strides) {
    a.sb = kv_strides[0]; a.sh = kv_strides[1]; a.sn = kv_strides[2];
    if (a.sb < 0 || a.sh < 0 || a.sn < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.sn = D;
    a.sh = (int64_t)N * D;
    a.sb = (int64_t)H * N * D;
  }
  if (D != 32 && D != 64 && D != 128) return GMLA_ERR_UNSUPPORTED;
  // 16-byte loads of 8 channels: rows must start 16-byte aligned
  const size_t es = elem_size(dtype);
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, es) ||
      (G && !aligned(G, es)) || (a.sb * es) % 16 || (a.sh * es) % 16 || (a.sn * es) % 16)
    return GMLA_ERR_INVALID_ARG;
  int splits = num_splits ? num_splits : gmla_decode_num_splits(B, H, N, D);
  if (splits > N) splits = N;
  a.splits = splits;
  a.ws = nullptr;
  if (splits > 1) {
    const size_t need = gmla_decode_workspace_bytes(B, H, N, D, splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GMLA_ERR_WORKSPACE;
    a.ws = (float*)workspace;
  }
  if (log_enabled())
    fprintf(stderr, "gmla: decode B=%d H=%d N=%d D=%d splits=%d\n", B, H, N, D, splits);
  return hip_status(launch_decode(dtype, a, (hipStream_t)stream));
}

int gmla_latent_expand(int dtype, int M, int d_c, int d_model, const void* C, const void* W_k,
                       const void* W_v, void* K, void* V, void* stream) {
  if (!valid_dtype(dtype) || M <= 0 || d_c <= 0 || d_model <= 0) return GMLA_ERR_INVALID_ARG;
  if (!C || !W_k || !W_v || !K || !V) return GMLA_ERR_INVALID_ARG;
  if (dtype == GMLA_BF16 &&
      (d_c % 8 || !aligned(C, 16) || !aligned(W_k, 16) || !aligned(W_v, 16) || !aligned(K, 2) ||
       !aligned(V, 2)))
    return GMLA_ERR_INVALID_ARG;
  if (dtype == GMLA_F32 && (!aligned(C, 4) || !aligned(W_k, 4) || !aligned(W_v, 4) ||
                            !aligned(K, 4) || !aligned(V, 4)))
    return GMLA_ERR_INVALID_ARG;
  GemmArgs p;
  p.M = M; p.N = d_model; p.K = d_c;
  p.x = C; p.w = W_k; p.w2 = W_v; p.N2 = d_model;
  p.g = nullptr; p.y = K; p.y2 = V;
  return hip_status(launch_gemm(dtype, p, (hipStream_t)stream));
}

int gmla_gate_out(int dtype, int M, int d_model, const void* G, const void* O_tilde,
                  const void* W_o, void* Y, void* stream) {
  if (!valid_dtype(dtype) || M <= 0 || d_model <= 0) return GMLA_ERR_INVALID_ARG;
  if (!O_tilde || !Y) return GMLA_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (!aligned(O_tilde, es) || !aligned(Y, es) || (G && !aligned(G, es)) ||
      (W_o && !aligned(W_o, es)))
    return GMLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (!W_o) return hip_status(launch_gate_only(dtype, (int64_t)M * d_model, G, O_tilde, Y, s));
  if (dtype == GMLA_BF16 &&
      (d_model % 8 || !aligned(O_tilde, 16) || !aligned(W_o, 16) || (G && !aligned(G, 16))))
    return GMLA_ERR_INVALID_ARG;
  GemmArgs p;
  p.M = M; p.N = d_model; p.K = d_model;
  p.x = O_tilde; p.w = W_o; p.w2 = nullptr; p.N2 = 0;
  p.g = G; p.y = Y; p.y2 = nullptr;
  return hip_status(launch_gemm(dtype, p, s));
}

int gmla_linear(int dtype, int M, int N, int K, const void* X, const void* W, void* Y,
                void* stream) {
  if (!valid_dtype(dtype) || M <= 0 || N <= 0 || K <= 0) return GMLA_ERR_INVALID_ARG;
  if (!X || !W || !Y) return GMLA_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (!aligned(X, es) || !aligned(W, es) || !aligned(Y, es)) return GMLA_ERR_INVALID_ARG;
  if (dtype == GMLA_BF16 && (K % 8 || !aligned(X, 16) || !aligned(W, 16)))
    return GMLA_ERR_INVALID_ARG;
  GemmArgs p;
  p.M = M; p.N = N; p.K = K;
  p.x = X; p.w = W; p.w2 = nullptr; p.N2 = 0;
  p.g = nullptr; p.y = Y; p.y2 = nullptr;
  return hip_status(launch_gemm(dtype, p, (hipStream_t)stream));
}

}  // extern "C"
