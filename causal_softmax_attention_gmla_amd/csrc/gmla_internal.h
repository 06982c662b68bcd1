// Internal declarations shared by the HIP translation units of libgmla.
// Device types and helpers for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmla {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator dies; workgroups are dealt round-robin

// log2(e): softmax is evaluated as 2^(x * scale * log2 e - m), using the hardware 2^x.
constexpr float kLog2e = 1.4426950408889634f;

// bf16 <-> f32 without library calls: bf16 is the top half of an IEEE float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16 x) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, x)) << 16);
}
// Round-to-nearest-even f32 -> bf16 (the compiler emits v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic sigmoid in f32: 1 / (1 + e^-x), with e^-x = 2^(-x log2 e).
__device__ __forceinline__ float sigmoidf_(float x) {
  return 1.0f / (1.0f + __expf(-x));
}

// Element loads/stores generic over float and bf16 storage.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16> {
  static __device__ __forceinline__ float load(const bf16* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(bf16* p, float v) { *p = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- launchers
// Each returns a hipError_t from the launch; arguments are already validated.

struct PrefillArgs {
  int B, T, H, D;         // T: query rows
  int Tk;                 // key rows (>= T); query i sits at position i + Tk - T
  float scale;
  int causal;
  const void *q, *k, *v;
  int64_t qsb, qst, qsh;  // element strides of Q (batch, token, head); d is contiguous
  int64_t sb, st, sh;     // element strides of K and V (batch, token, head)
  const void* g;          // nullable gate logits [B, T, H*D]
  void* o;                // [B, T, H*D]
};
hipError_t launch_prefill_bf16_mfma(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_simple_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_simple_bf16(const PrefillArgs& a, hipStream_t s);

struct DecodeArgs {
  int B, H, N, D;
  float scale;
  const void *q, *k, *v;
  int64_t sb, sh, sn;  // K/V element strides (batch, head, key); d contiguous
  const void* g;       // nullable [B, H*D]
  void* o;             // [B, H*D]
  float* ws;           // [B, H, splits, D + 2] partials (m, l, o[D]); NULL when splits == 1
  int splits;
};
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s);

struct GemmArgs {
  int M, N, K;
  const void* x;   // [M, K]
  const void* w;   // [N, K]            (first weight)
  const void* w2;  // [N2, K] or NULL   (second weight: columns N..N+N2 of the product)
  int N2;
  const void* g;   // nullable gate logits [M, K]: A operand = sigmoid(g) * x
  void* y;         // [M, N]
  void* y2;        // [M, N2] or NULL
};
hipError_t launch_gemm(int dtype, const GemmArgs& a, hipStream_t s);
// LDS-direct pipelined bf16 GEMM: no gate, K a multiple of 64, N (and N2) a multiple
// of 8, 16-byte aligned operands, 8-byte aligned outputs.
bool gemm_lds_supported(const GemmArgs& a);
hipError_t launch_gemm_lds(const GemmArgs& a, hipStream_t s);
hipError_t launch_gate_only(int dtype, int64_t n, const void* g, const void* x, void* y,
                            hipStream_t s);

}  // namespace gmla
