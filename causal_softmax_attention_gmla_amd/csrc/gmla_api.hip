// C ABI of libgmla: argument validation on the host, kernel choice, launch.
// Every check runs before any HIP call, so a bad argument never touches the device.
#include "../../include/gmla.h"

#include <stdio.h>
#include <stdlib.h>

#include <mutex>
#include <utility>

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
    case GMLA_ERR_TOO_LARGE: return "GMLA_ERR_TOO_LARGE";
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
  if (Tk > kMaxKeys) return GMLA_ERR_UNSUPPORTED;
  PrefillArgs a;
  a.B = B; a.T = Tq; a.Tk = Tk; a.H = H; a.D = D;
  a.scale = scale;
  a.causal = causal;
  a.q = Q; a.k = K; a.v = V; a.g = G; a.o = O;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
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

int gmla_attend_varlen(int dtype, int B, int H, int D, float scale, int causal, const void* Q,
                       const int64_t* q_strides, const int* cu_seqlens_q, int max_seqlen_q,
                       const void* K, const void* V, const int64_t* kv_strides,
                       const int* cu_seqlens_k, int max_seqlen_k, const void* G, void* O,
                       void* stream) {
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || D <= 0 || max_seqlen_q <= 0 || max_seqlen_k < 0)
    return GMLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GMLA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O || !cu_seqlens_q || !cu_seqlens_k) return GMLA_ERR_INVALID_ARG;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4)) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  if (max_seqlen_q > kMaxKeys || max_seqlen_k > kMaxKeys) return GMLA_ERR_UNSUPPORTED;
  PrefillArgs a;
  a.B = B; a.T = max_seqlen_q; a.Tk = max_seqlen_k; a.H = H; a.D = D;
  a.scale = scale;
  a.causal = causal;
  a.q = Q; a.k = K; a.v = V; a.g = G; a.o = O;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.qsb = a.sb = 0;  // packed rows: the sequence offsets replace the batch strides
  if (q_strides) {
    a.qst = q_strides[0]; a.qsh = q_strides[1];
    if (a.qst < 0 || a.qsh < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.qsh = D;
    a.qst = (int64_t)H * D;
  }
  if (kv_strides) {
    a.st = kv_strides[0]; a.sh = kv_strides[1];
    if (a.st < 0 || a.sh < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.sh = D;
    a.st = (int64_t)H * D;
  }
  const size_t es = elem_size(dtype);
  if (!aligned(Q, es) || !aligned(K, es) || !aligned(V, es) || !aligned(O, es) ||
      (G && !aligned(G, es)))
    return GMLA_ERR_INVALID_ARG;
  if (D != 32 && D != 64 && D != 128) return GMLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == GMLA_BF16 && D == 128) {
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
        (G && !aligned(G, 16)) || a.st % 8 || a.sh % 8 || a.qst % 8 || a.qsh % 8)
      return GMLA_ERR_INVALID_ARG;
    if (a.st >= (int64_t)1 << 24) return GMLA_ERR_UNSUPPORTED;
    if (log_enabled())
      fprintf(stderr, "gmla: varlen bf16 mfma B=%d max Tq=%d max Tk=%d H=%d causal=%d\n", B,
              max_seqlen_q, max_seqlen_k, H, causal);
    e = launch_prefill_bf16_varlen(a, s);
  } else if (dtype == GMLA_BF16) {
    e = launch_prefill_simple_bf16(a, s);
  } else {
    e = launch_prefill_simple_f32(a, s);
  }
  return hip_status(e);
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

}  // extern "C"

namespace {

// Validation shared by the decode entry points: fills `a` (all but the workspace) and
// the split count.  Returns GMLA_OK or the status the call must return.
int decode_prepare(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                   const void* K, const void* V, const int64_t* kv_strides, const void* G,
                   void* O, int num_splits, DecodeArgs& a) {
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 || D <= 0) return GMLA_ERR_INVALID_ARG;
  if (!Q || !K || !V || !O) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 4096) return GMLA_ERR_INVALID_ARG;
  // key indices are 32-bit in the kernel: leave room for one step of 1024 rows
  if (N > kMaxKeys) return GMLA_ERR_UNSUPPORTED;
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
  a.lens = nullptr;
  return GMLA_OK;
}

}  // namespace

extern "C" {

int gmla_attend_decode(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                       const void* K, const void* V, const int64_t* kv_strides, const void* G,
                       void* O, void* workspace, size_t workspace_bytes, int num_splits,
                       void* stream) {
  DecodeArgs a;
  const int st = decode_prepare(dtype, B, H, N, D, scale, Q, K, V, kv_strides, G, O, num_splits, a);
  if (st != GMLA_OK) return st;
  if (a.splits > 1) {
    const size_t need = gmla_decode_workspace_bytes(B, H, N, D, a.splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GMLA_ERR_WORKSPACE;
    a.ws = (float*)workspace;
  }
  if (log_enabled())
    fprintf(stderr, "gmla: decode B=%d H=%d N=%d D=%d splits=%d\n", B, H, N, D, a.splits);
  return hip_status(launch_decode(dtype, a, (hipStream_t)stream));
}

int gmla_attend_decode_varlen(int dtype, int B, int H, int N, int D, float scale, const void* Q,
                              const void* K, const void* V, const int64_t* kv_strides,
                              const int* kv_lens, const void* G, void* O, void* workspace,
                              size_t workspace_bytes, int num_splits, void* stream) {
  if (!kv_lens || !aligned(kv_lens, 4)) return GMLA_ERR_INVALID_ARG;
  DecodeArgs a;
  const int st = decode_prepare(dtype, B, H, N, D, scale, Q, K, V, kv_strides, G, O, num_splits, a);
  if (st != GMLA_OK) return st;
  a.lens = kv_lens;
  if (a.splits > 1) {
    const size_t need = gmla_decode_workspace_bytes(B, H, N, D, a.splits);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return GMLA_ERR_WORKSPACE;
    a.ws = (float*)workspace;
  }
  if (log_enabled())
    fprintf(stderr, "gmla: decode varlen B=%d H=%d N<=%d D=%d splits=%d\n", B, H, N, D, a.splits);
  return hip_status(launch_decode(dtype, a, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------- decode without allocation
// For callers that cannot allocate (code under HIP graph capture, tight serving loops):
// the split partials live in a fixed device array instead of a caller workspace.  Host
// code never passes the array's name to a kernel (that is a host-side stand-in, not a
// device address): the device address is looked up once per device, with that device
// current, and kept.
namespace {

constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_scratch_lock;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on first use).
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GMLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GMLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_lock);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GMLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GMLA_OK;
}

}  // namespace

extern "C" {

size_t gmla_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gmla_attend_decode_noalloc(int dtype, int B, int H, int N, int D, float scale,
                               const void* Q, const void* K, const void* V,
                               const int64_t* kv_strides, const void* G, void* O, int num_splits,
                               void* stream) {
  DecodeArgs a;
  const int st = decode_prepare(dtype, B, H, N, D, scale, Q, K, V, kv_strides, G, O, num_splits, a);
  if (st != GMLA_OK) return st;
  if (a.splits > 1) {
    if (gmla_decode_workspace_bytes(B, H, N, D, a.splits) > kScratchBytes) return GMLA_ERR_TOO_LARGE;
    void* p = nullptr;
    const int sst = scratch_on_current_device(&p);
    if (sst != GMLA_OK) return sst;
    // every (batch, head, split) slot is written before the merge reads it: no clearing
    a.ws = (float*)p;
  }
  if (log_enabled())
    fprintf(stderr, "gmla: decode (no alloc) B=%d H=%d N=%d D=%d splits=%d\n", B, H, N, D,
            a.splits);
  return hip_status(launch_decode(dtype, a, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------- decode over the latent cache
namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Key ranges of the latent decode: kps rows each (a multiple of the 32-row tile), and the
// number of ranges that then covers N with none empty.
void latent_plan(int B, int H, int N, int num_splits, int* splits, int* kps) {
  long s = num_splits;
  if (s <= 0) {
    // about 512 workgroups of 32 heads, but ranges of at least 128 rows: each range's
    // partials (d_c + 2 floats per head) cost about what 32 latent rows do
    const long groups = (long)B * ((H + 31) / 32);
    s = (512 + groups - 1) / groups;
    long cap = N / 128;
    if (cap < 1) cap = 1;
    if (s > cap) s = cap;
  }
  if (s > N) s = N;
  if (s > 1024) s = 1024;  // the merge keeps one weight per range in LDS
  if (s < 1) s = 1;
  long k = ((long)N + s - 1) / s;
  k = (k + 31) / 32 * 32;
  *kps = (int)k;
  *splits = (int)(((long)N + k - 1) / k);
}

size_t latent_ws_bytes(int B, int H, int d_c, int splits) {
  const size_t heads = (size_t)B * H;
  return round256(heads * d_c * 2) + round256(heads * splits * 2 * sizeof(float)) +
         heads * splits * d_c * sizeof(float);
}

}  // namespace

extern "C" {

int gmla_decode_latent_num_splits(int B, int H, int N, int d_c) {
  (void)d_c;
  if (B <= 0 || H <= 0 || N <= 0) return 1;
  int splits, kps;
  latent_plan(B, H, N, 0, &splits, &kps);
  return splits;
}

size_t gmla_decode_latent_workspace_bytes(int B, int H, int N, int d_c, int num_splits) {
  if (B <= 0 || H <= 0 || N <= 0 || d_c <= 0 || num_splits < 0) return 0;
  int splits, kps;
  latent_plan(B, H, N, num_splits, &splits, &kps);
  return latent_ws_bytes(B, H, d_c, splits);
}

}  // extern "C"

namespace {

int decode_latent_impl(int dtype, int B, int H, int N, int D, int d_c, float scale,
                       const void* Q, const void* C, const int64_t* c_strides, const int* lens,
                       const void* W_k, const void* W_v, const void* G, void* O,
                       void* workspace, size_t workspace_bytes, int num_splits, void* stream) {
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 || D <= 0 || d_c <= 0)
    return GMLA_ERR_INVALID_ARG;
  if (!Q || !C || !W_k || !W_v || !O) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  if (num_splits < 0) return GMLA_ERR_INVALID_ARG;
  LatentDecodeArgs a;
  if (c_strides) {
    a.csb = c_strides[0];
    a.csn = c_strides[1];
    if (a.csb < 0 || a.csn < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.csn = d_c;
    a.csb = (int64_t)N * d_c;
  }
  if (!aligned(O, 2) || (G && !aligned(G, 2)) || !aligned(Q, 16) || !aligned(C, 16) ||
      !aligned(W_k, 16) || !aligned(W_v, 16) || a.csb % 8 || a.csn % 8)
    return GMLA_ERR_INVALID_ARG;
  if (dtype != GMLA_BF16 || D != 128 || (d_c != 128 && d_c != 256 && d_c != 512))
    return GMLA_ERR_UNSUPPORTED;
  // grid limits (heads and batch rows are grid dimensions), 32-bit row indices, and 32-bit
  // byte offsets inside one 32-row tile
  if (N > kMaxKeys || B > 65535 || H > 65535 || a.csn >= ((int64_t)1 << 25))
    return GMLA_ERR_UNSUPPORTED;
  latent_plan(B, H, N, num_splits, &a.splits, &a.kps);
  const size_t heads = (size_t)B * H;
  const size_t need = latent_ws_bytes(B, H, d_c, a.splits);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return GMLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  a.qp = (bf16*)ws;
  a.ml = (float*)(ws + round256(heads * d_c * 2));
  a.u = (float*)(ws + round256(heads * d_c * 2) + round256(heads * a.splits * 2 * sizeof(float)));
  a.B = B; a.H = H; a.N = N; a.DC = d_c;
  a.q = (const bf16*)Q;
  a.c = (const bf16*)C;
  a.wk = (const bf16*)W_k;
  a.wv = (const bf16*)W_v;
  a.g = (const bf16*)G;
  a.o = (bf16*)O;
  a.c2 = scale * kLog2e;
  a.lens = lens;
  if (log_enabled())
    fprintf(stderr, "gmla: decode latent B=%d H=%d N=%d d_c=%d splits=%d (%d rows each)%s\n", B,
            H, N, d_c, a.splits, a.kps, lens ? " per-row lengths" : "");
  return hip_status(launch_decode_latent(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int gmla_attend_decode_latent(int dtype, int B, int H, int N, int D, int d_c, float scale,
                              const void* Q, const void* C, const int64_t* c_strides,
                              const void* W_k, const void* W_v, const void* G, void* O,
                              void* workspace, size_t workspace_bytes, int num_splits,
                              void* stream) {
  return decode_latent_impl(dtype, B, H, N, D, d_c, scale, Q, C, c_strides, nullptr, W_k, W_v, G,
                            O, workspace, workspace_bytes, num_splits, stream);
}

int gmla_attend_decode_latent_varlen(int dtype, int B, int H, int N, int D, int d_c, float scale,
                                     const void* Q, const void* C, const int64_t* c_strides,
                                     const int* kv_lens, const void* W_k, const void* W_v,
                                     const void* G, void* O, void* workspace,
                                     size_t workspace_bytes, int num_splits, void* stream) {
  if (!kv_lens || !aligned(kv_lens, 4)) return GMLA_ERR_INVALID_ARG;
  return decode_latent_impl(dtype, B, H, N, D, d_c, scale, Q, C, c_strides, kv_lens, W_k, W_v, G,
                            O, workspace, workspace_bytes, num_splits, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- latent-fused prefill
namespace {

struct LatentPrefillLayout {
  size_t kv_bytes;  // one of K, V
  size_t flag_ints;
  size_t total;
};

LatentPrefillLayout latent_prefill_layout(int B, int T, int H, int D) {
  LatentPrefillLayout l;
  l.kv_bytes = round256((size_t)B * T * H * D * 2);
  const size_t nE = ((size_t)T + 127) / 128;
  l.flag_ints = (size_t)B * H * nE + kNumXcd + 1;  // ready flags, per-XCD counters, error word
  l.total = 2 * l.kv_bytes + l.flag_ints * sizeof(int);
  return l;
}

}  // namespace

extern "C" {

size_t gmla_prefill_latent_workspace_bytes(int B, int T, int H, int D) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0) return 0;
  return latent_prefill_layout(B, T, H, D).total;
}

int gmla_attend_prefill_latent(int dtype, int B, int T, int H, int D, int d_c, float scale,
                               int causal, const void* Q, const int64_t* q_strides, const void* C,
                               const void* W_k, const void* W_v, const void* G, void* O,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype) || B <= 0 || T <= 0 || H <= 0 || D <= 0 || d_c <= 0)
    return GMLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GMLA_ERR_INVALID_ARG;
  if (!Q || !C || !W_k || !W_v || !O) return GMLA_ERR_INVALID_ARG;
  if (!(scale == scale) || scale <= 0.0f) return GMLA_ERR_INVALID_ARG;
  LatentPrefillArgs f;
  PrefillArgs& a = f.p;
  if (q_strides) {
    a.qsb = q_strides[0]; a.qst = q_strides[1]; a.qsh = q_strides[2];
    if (a.qsb < 0 || a.qst < 0 || a.qsh < 0) return GMLA_ERR_INVALID_ARG;
  } else {
    a.qsh = D;
    a.qst = (int64_t)H * D;
    a.qsb = (int64_t)T * H * D;
  }
  if (!aligned(Q, 16) || !aligned(C, 16) || !aligned(W_k, 16) || !aligned(W_v, 16) ||
      !aligned(O, 16) || (G && !aligned(G, 16)) || a.qsb % 8 || a.qst % 8 || a.qsh % 8)
    return GMLA_ERR_INVALID_ARG;
  if (dtype != GMLA_BF16 || D != 128 || d_c % 32 || d_c > (1 << 20)) return GMLA_ERR_UNSUPPORTED;
  if (T > kMaxKeys || (int64_t)H * D >= ((int64_t)1 << 24)) return GMLA_ERR_UNSUPPORTED;
  const LatentPrefillLayout l = latent_prefill_layout(B, T, H, D);
  const int64_t nE = ((int64_t)T + 127) / 128;
  if ((int64_t)B * H * nE * 2 > 0x7fffffffLL) return GMLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < l.total || !aligned(workspace, 256)) return GMLA_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  f.kws = (bf16*)ws;
  f.vws = (bf16*)(ws + l.kv_bytes);
  f.flags = (int*)(ws + 2 * l.kv_bytes);
  f.ntasks_e = (int)(B * H * nE);
  f.counter = f.flags + f.ntasks_e;
  f.error = f.flags + f.ntasks_e + kNumXcd;
  f.nE = (int)nE;
  f.nqb = (int)nE;  // 128-query blocks, 128-row expansion blocks
  f.ntasks = f.ntasks_e + B * H * f.nqb;
  f.c = (const bf16*)C;
  f.wk = (const bf16*)W_k;
  f.wv = (const bf16*)W_v;
  f.DC = d_c;
  a.B = B; a.T = T; a.Tk = T; a.H = H; a.D = D;
  a.scale = scale;
  a.causal = causal;
  a.q = Q; a.k = f.kws; a.v = f.vws; a.g = G; a.o = O;
  a.sh = D;
  a.st = (int64_t)H * D;
  a.sb = (int64_t)T * H * D;
  a.cu_q = nullptr;
  a.cu_k = nullptr;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return GMLA_ERR_HIP;
  // the task queues are per XCD: the device must expose all eight of them (one partition)
  if (cus % kNumXcd || cus < 32 * kNumXcd) return GMLA_ERR_UNSUPPORTED;
  if (log_enabled())
    fprintf(stderr, "gmla: prefill latent B=%d T=%d H=%d d_c=%d tasks=%d+%d workgroups=%d\n", B, T,
            H, d_c, f.ntasks_e, f.ntasks - f.ntasks_e, 2 * cus);
  return hip_status(launch_prefill_latent(f, 2 * cus, (hipStream_t)stream));
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

extern "C" {

size_t gmla_linear_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  int splits, kps;
  gemm_splitk_plan(M, N, K, &splits, &kps);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

int gmla_linear_ws(int dtype, int M, int N, int K, const void* X, const void* W, void* Y,
                   void* workspace, size_t workspace_bytes, void* stream) {
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
  hipStream_t s = (hipStream_t)stream;
  int splits = 1, kps = 0;
  if (dtype == GMLA_BF16) gemm_splitk_plan(M, N, K, &splits, &kps);
  const size_t need = (size_t)splits * M * N * sizeof(float);
  // the split path needs 16-byte rows everywhere and the partials' space; otherwise the
  // call is gmla_linear
  if (splits > 1 && workspace && workspace_bytes >= need && aligned(workspace, 16) &&
      aligned(Y, 16) && (int64_t)128 * K * 2 < ((int64_t)1 << 31)) {
    p.part = (float*)workspace;
    p.splits = splits;
    p.kps = kps;
    if (log_enabled())
      fprintf(stderr, "gmla: linear split-K M=%d N=%d K=%d ranges=%d (%d stages each)\n", M, N, K,
              splits, kps);
    return hip_status(launch_gemm_splitk(p, s));
  }
  return hip_status(launch_gemm(dtype, p, s));
}

// The gated bf16 projection through the LDS-pipelined GEMM: the gate kernel writes
// sigmoid(G) (.) O~ (rounded to bf16, exactly the operand the gate prologue forms) to the
// workspace, which is then the GEMM's A operand.  Zero when the shape does not take it.
size_t gmla_gate_out_workspace_bytes(int dtype, int M, int d_model) {
  if (dtype != GMLA_BF16 || M <= 0 || d_model <= 0 || d_model % 64) return 0;
  if ((int64_t)256 * d_model * 2 >= ((int64_t)1 << 31)) return 0;
  return (size_t)M * d_model * 2;
}

int gmla_gate_out_ws(int dtype, int M, int d_model, const void* G, const void* O_tilde,
                     const void* W_o, void* Y, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const size_t need = gmla_gate_out_workspace_bytes(dtype, M, d_model);
  if (!G || !W_o || need == 0 || !workspace || workspace_bytes < need ||
      !aligned(workspace, 16) || !O_tilde || !Y || !aligned(O_tilde, 16) || !aligned(G, 16) ||
      !aligned(W_o, 16) || !aligned(Y, 16))
    return gmla_gate_out(dtype, M, d_model, G, O_tilde, W_o, Y, stream);
  // the workspace may not overlap an input or the output (it is written while they are read)
  const auto span = [](const void* p, size_t n) {
    return std::make_pair((uintptr_t)p, (uintptr_t)p + n);
  };
  const auto ws = span(workspace, need);
  const size_t mat = (size_t)M * d_model * 2;
  for (auto o : {span(G, mat), span(O_tilde, mat), span(W_o, (size_t)d_model * d_model * 2),
                 span(Y, mat)})
    if (ws.first < o.second && o.first < ws.second) return GMLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  GemmArgs p;
  p.M = M; p.N = d_model; p.K = d_model;
  p.x = workspace; p.w = W_o; p.w2 = nullptr; p.N2 = 0;
  p.g = nullptr; p.y = Y; p.y2 = nullptr;
  if (!gemm_lds_supported(p)) return gmla_gate_out(dtype, M, d_model, G, O_tilde, W_o, Y, stream);
  const hipError_t e = launch_gate_only(dtype, (int64_t)M * d_model, G, O_tilde, workspace, s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_gemm_lds(p, s));
}

}  // extern "C"
