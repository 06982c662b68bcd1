// Decode: one query per (batch, head) against N cached keys, all visible (the query
// sits at position N - 1: "Kimi K3 - Softmax over keys", decode at p = 1000 with
// 1001 keys; "Kimi K2 - Construct causal mask", positions continue from the cached
// length).
//
// The work is streaming: each key and value row is read once from HBM, so the
// kernel is laid out for bandwidth, not for the matrix cores:
//  * Grid (split, head, batch).  A split is a contiguous key range; inside it each
//    of the 4 waves streams its own contiguous run of 8 x (64 / (D/8)) rows per step
//    with 16-byte loads, all 16 loads of a lane issued before any is used.  The loads
//    are non-temporal: every byte of the cache is read once, so keeping it in the
//    caches only evicts other data (measured: 5.5 -> 6.3-6.4 TB/s at 1001 keys,
//    6.2 -> 7.0 TB/s at 131072 keys, against about 7.05 TB/s for a plain read stream).
//  * A lane owns 8 channels of one key row; the q.k dot product is reduced over the
//    D/8 lanes of the row with DPP row operations (no LDS).
//  * Online softmax in base 2 per lane (running max m, sum l, 8 output channels),
//    merged across the lanes of a wave, across waves through LDS, and across splits
//    by log-sum-exp: m = max_j m_j, l = sum_j l_j 2^(m_j - m),
//    o = sum_j o_j 2^(m_j - m) / l -- an exact regrouping of the one softmax over all
//    keys ("Kimi K3 - Softmax over keys", the formula).
//  * Per-row cache lengths (an optional device array): row b holds its own number of
//    keys, and its query sits at position lens[b] - 1; the key ranges are those of the
//    longest row, so a shorter row's later ranges are empty (m = -inf, weight 0).
//  * With one split the workgroup writes the final (normalised, optionally gated)
//    output itself; otherwise it writes (m, l, o) to the workspace and a small merge
//    kernel finishes.
#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int NT = 256;  // 4 waves
constexpr int U = 8;     // key rows per lane per step

template <typename T> struct Row8;
template <> struct Row8<bf16> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16* p) {
    w = __builtin_nontemporal_load((const u32x4*)p);
  }
  __device__ __forceinline__ void zero() { w = u32x4{}; }
  __device__ __forceinline__ float at(int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
};
template <> struct Row8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load((const f32x4*)p);
    b = __builtin_nontemporal_load((const f32x4*)(p + 4));
  }
  __device__ __forceinline__ void zero() { a = f32x4{}; b = f32x4{}; }
  __device__ __forceinline__ float at(int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

// DPP lane permutations within a row of 16 lanes.
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false);
  return x + __int_as_float(y);
}

// Sum over the LPK consecutive lanes that hold one key row (LPK = 4, 8 or 16).
template <int LPK>
__device__ __forceinline__ float row_sum(float x) {
  x = dpp_add<kQuadSwap1>(x);
  x = dpp_add<kQuadSwap2>(x);
  if (LPK >= 8) x = dpp_add<kRowHalfMirror>(x);
  if (LPK >= 16) x = dpp_add<kRowMirror>(x);
  return x;
}

struct Partial {
  float m, l, o[8];
};

// Merge partial b into a (log-sum-exp regrouping); empty partials have m = -inf.
__device__ __forceinline__ void merge_into(Partial& a, const Partial& b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return;
  const float fa = a.m == -INFINITY ? 0.0f : fast_exp2(a.m - m);
  const float fb = b.m == -INFINITY ? 0.0f : fast_exp2(b.m - m);
  a.l = a.l * fa + b.l * fb;
#pragma unroll
  for (int e = 0; e < 8; ++e) a.o[e] = a.o[e] * fa + b.o[e] * fb;
  a.m = m;
}

__device__ __forceinline__ Partial shfl_partial(const Partial& p, int mask) {
  Partial r;
  r.m = __shfl_xor(p.m, mask);
  r.l = __shfl_xor(p.l, mask);
#pragma unroll
  for (int e = 0; e < 8; ++e) r.o[e] = __shfl_xor(p.o[e], mask);
  return r;
}

template <typename T, int D, bool LENS>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecodeArgs a, int keys_per_split) {
  constexpr int LPK = D / 8;      // lanes per key row
  constexpr int KPW = 64 / LPK;   // key rows per wave per load
  constexpr int WSTEP = KPW * U;  // key rows per wave per step
  __shared__ Partial red[4][LPK];

  const int split = blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c8 = lane % LPK;  // channel chunk: channels 8*c8 .. 8*c8+7
  const int kr = lane / LPK;  // key row within a load

  // with per-row cache lengths, row b holds lens[b] keys (clamped to [0, N]) and its query
  // sits at position lens[b] - 1
  const int nb = LENS ? min(max(a.lens[b], 0), a.N) : a.N;
  const int n0 = split * keys_per_split;
  const int n1 = min(nb, n0 + keys_per_split);
  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const T* Kh = (const T*)a.k + head_off + c8 * 8;
  const T* Vh = (const T*)a.v + head_off + c8 * 8;

  float q[8];
  {
    Row8<T> qr;
    qr.load((const T*)a.q + ((int64_t)b * a.H + h) * D + c8 * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = qr.at(e);
  }
  const float c2 = a.scale * kLog2e;

  Partial st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = 0.0f;

  for (int base = n0 + wave * WSTEP; base < n1; base += 4 * WSTEP) {
    Row8<T> kf[U], vf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = base + u * KPW + kr;
      if (n < n1) {
        kf[u].load(Kh + (int64_t)n * a.sn);
        vf[u].load(Vh + (int64_t)n * a.sn);
      } else {
        kf[u].zero();
        vf[u].zero();
      }
    }
    float s[U];
    float mx = st.m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(q[e], kf[u].at(e), dot);
      dot = row_sum<LPK>(dot);
      s[u] = (base + u * KPW + kr < n1) ? dot * c2 : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    if (mx == -INFINITY) continue;  // no key of this lane in range
    const float alpha = fast_exp2(st.m - mx);  // st.m = -inf: alpha = 0
    st.l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[e] *= alpha;
    st.m = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = fast_exp2(s[u] - mx);
      st.l += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.o[e] = __builtin_fmaf(p, vf[u].at(e), st.o[e]);
    }
  }

  // merge the KPW key rows of the wave (lanes with the same channel chunk)
#pragma unroll
  for (int mask = LPK; mask < 64; mask <<= 1) merge_into(st, shfl_partial(st, mask));
  if (kr == 0) red[wave][c8] = st;
  __syncthreads();
  if (wave != 0 || kr != 0) return;
  Partial tot = red[0][c8];
#pragma unroll
  for (int w = 1; w < 4; ++w) merge_into(tot, red[w][c8]);

  if (a.splits == 1) {
    const int64_t row = ((int64_t)b * a.H + h) * D + c8 * 8;
    // (an empty cache row, possible only with per-row lengths, gives zeros)
    const float inv = (LENS && tot.l == 0.0f) ? 0.0f : 1.0f / tot.l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = tot.o[e] * inv;
      if (a.g) v *= sigmoidf_(Elem<T>::load((const T*)a.g + row + e));
      Elem<T>::store((T*)a.o + row + e, v);
    }
  } else {
    float* ws = a.ws + (((int64_t)b * a.H + h) * a.splits + split) * (D + 2);
    if (c8 == 0) {
      ws[0] = tot.m;
      ws[1] = tot.l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ws[2 + c8 * 8 + e] = tot.o[e];
  }
}

// One workgroup per (batch, head), one lane per channel.
template <typename T, int D, bool LENS>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* ws = a.ws + ((int64_t)b * a.H + h) * a.splits * (D + 2);
  float m = -INFINITY;
  for (int j = 0; j < a.splits; ++j) m = fmaxf(m, ws[j * (D + 2)]);
  float l = 0.0f, o = 0.0f;
  for (int j = 0; j < a.splits; ++j) {
    const float mj = ws[j * (D + 2)];
    if (mj == -INFINITY) continue;
    const float f = fast_exp2(mj - m);
    l = __builtin_fmaf(ws[j * (D + 2) + 1], f, l);
    o = __builtin_fmaf(ws[j * (D + 2) + 2 + d], f, o);
  }
  const int64_t idx = ((int64_t)b * a.H + h) * D + d;
  float v = (LENS && l == 0.0f) ? 0.0f : o / l;
  if (a.g) v *= sigmoidf_(Elem<T>::load((const T*)a.g + idx));
  Elem<T>::store((T*)a.o + idx, v);
}

template <typename T, int D, bool LENS>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const int kps = (a.N + a.splits - 1) / a.splits;
  hipLaunchKernelGGL((decode_split_kernel<T, D, LENS>), dim3(a.splits, a.H, a.B), dim3(NT), 0, s,
                     a, kps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D, LENS>), dim3(a.H, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_l(const DecodeArgs& a, hipStream_t s) {
  return a.lens ? launch_decode_t<T, D, true>(a, s) : launch_decode_t<T, D, false>(a, s);
}

}  // namespace

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) {
  const bool bf = dtype == 1;
  switch (a.D) {
    case 32: return bf ? launch_decode_l<bf16, 32>(a, s) : launch_decode_l<float, 32>(a, s);
    case 64: return bf ? launch_decode_l<bf16, 64>(a, s) : launch_decode_l<float, 64>(a, s);
    case 128: return bf ? launch_decode_l<bf16, 128>(a, s) : launch_decode_l<float, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmla
