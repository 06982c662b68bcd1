// Causal softmax attention on the vector ALUs in true float32 (no reduced-precision
// shortcut), for float32 tensors and for head widths the MFMA kernel does not take.
//
// Same definition as the MFMA kernel ("Gated MLA", section "Start from familiar
// attention"; "Kimi K3 - Softmax over keys"; "Kimi K2 - Construct causal mask"),
// with the optional channel-wise sigmoid gate ("Gated MLA", section "The
// channel-wise output gate").
//
// Queries may be the last rows of a longer key sequence (a chunk after a cache): query
// i then sits at position i + Tk - T ("Kimi K2 - Construct causal mask": positions
// continue from the cached length).
//
// One 64-lane workgroup takes 64 / TPQ queries of one (batch, head); each query is
// owned by TPQ lanes that split its head channels (DP channels each).  Key and value
// tiles of 64 rows are staged in LDS as float32; every lane keeps its query slice,
// its output slice and a running (max, sum) in registers, and writes the tile's
// scores to its own LDS row, so the softmax runs tile by tile with one rescale per
// tile.  exp is the accurate library expf.
#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int KT = 64;  // keys per tile

template <typename E, int D, int TPQ, bool VARLEN>
__global__ __launch_bounds__(64) void prefill_simple_kernel(PrefillArgs a) {
  constexpr int DP = D / TPQ;    // channels per lane
  constexpr int QPB = 64 / TPQ;  // queries per workgroup
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  __shared__ float ss[QPB][KT + 1];

  const int nqb = (a.T + QPB - 1) / QPB;
  const int head_lin = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int b = head_lin / a.H, h = head_lin % a.H;
  const int tid = threadIdx.x;
  const int qi = tid % QPB;   // query slot in the workgroup
  const int part = tid / QPB;  // channel slice
  const int t = qb * QPB + qi;
  // per-sequence lengths: sequence b owns packed query rows cu_q[b] .. and key rows
  // cu_k[b] ..; its query i sits at position i + Tk_b - Tq_b
  int T, Tk;
  int64_t qrow0;
  const E *Qh, *Kh, *Vh;
  if (VARLEN) {
    const int qlo = a.cu_q[b], klo = a.cu_k[b];
    T = a.cu_q[b + 1] - qlo;
    Tk = max(a.cu_k[b + 1] - klo, 0);
    if (qb * QPB >= T) return;  // the whole workgroup: past this sequence's end
    qrow0 = qlo;
    Qh = (const E*)a.q + (int64_t)qlo * a.qst + (int64_t)h * a.qsh;
    Kh = (const E*)a.k + (int64_t)klo * a.st + (int64_t)h * a.sh;
    Vh = (const E*)a.v + (int64_t)klo * a.st + (int64_t)h * a.sh;
  } else {
    T = a.T;
    Tk = a.Tk;
    qrow0 = (int64_t)b * a.T;
    const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
    Qh = (const E*)a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh;
    Kh = (const E*)a.k + head_off;
    Vh = (const E*)a.v + head_off;
  }
  const int off = Tk - T;

  float q[DP], o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    q[i] = t < T ? Elem<E>::load(Qh + (int64_t)t * a.qst + part * DP + i) : 0.0f;
    o[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  // query t sits at position t + off: it sees keys up to there (causal) or all of them
  const int last_visible = a.causal ? min(t + off, Tk - 1) : Tk - 1;
  const int block_last = a.causal ? min(qb * QPB + QPB - 1 + off, Tk - 1) : Tk - 1;

  for (int k0 = 0; k0 <= block_last; k0 += KT) {
    __syncthreads();
    for (int idx = tid; idx < KT * D; idx += 64) {
      const int r = idx / D, c = idx % D;
      const int key = k0 + r;
      ks[r][c] = key < Tk ? Elem<E>::load(Kh + (int64_t)key * a.st + c) : 0.0f;
      vs[r][c] = key < Tk ? Elem<E>::load(Vh + (int64_t)key * a.st + c) : 0.0f;
    }
    __syncthreads();
    // scores of this tile; keys after the query (or past the end) get -inf
    float mt = -INFINITY;
    for (int r = 0; r < KT; ++r) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < DP; ++i) dot = __builtin_fmaf(q[i], ks[r][part * DP + i], dot);
      if (TPQ == 2) dot += __shfl_xor(dot, 32);
      const float sc = (k0 + r <= last_visible) ? dot * a.scale : -INFINITY;
      if (part == 0) ss[qi][r] = sc;
      mt = fmaxf(mt, sc);
    }
    __syncthreads();
    const float mnew = fmaxf(m, mt);
    if (mnew == -INFINITY) continue;  // nothing visible yet (only past-the-end rows)
    const float alpha = expf(m - mnew);  // m = -inf on the first tile: alpha = 0
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) o[i] *= alpha;
    m = mnew;
    for (int r = 0; r < KT; ++r) {
      const float p = expf(ss[qi][r] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) o[i] = __builtin_fmaf(p, vs[r][part * DP + i], o[i]);
    }
  }
  if (t >= T) return;
  const int64_t row = (qrow0 + t) * ((int64_t)a.H * D) + (int64_t)h * D + part * DP;
  const E* g = a.g ? (const E*)a.g + row : nullptr;
  E* out = (E*)a.o + row;
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    // a query that sees no key (possible only with per-sequence lengths) writes zeros
    float v = (VARLEN && l == 0.0f) ? 0.0f : o[i] / l;
    if (g) v *= 1.0f / (1.0f + expf(-Elem<E>::load(g + i)));
    Elem<E>::store(out + i, v);
  }
}

template <typename E, bool VARLEN>
hipError_t launch_simple(const PrefillArgs& a, hipStream_t s) {
  auto go = [&](auto kernel, int qpb) {
    const long nqb = (a.T + qpb - 1) / qpb;
    const long grid = nqb * a.B * a.H;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(64), 0, s, a);
    return hipGetLastError();
  };
  switch (a.D) {
    case 32: return go(prefill_simple_kernel<E, 32, 1, VARLEN>, 64);
    case 64: return go(prefill_simple_kernel<E, 64, 1, VARLEN>, 64);
    case 128: return go(prefill_simple_kernel<E, 128, 2, VARLEN>, 32);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_simple_f32(const PrefillArgs& a, hipStream_t s) {
  return a.cu_q ? launch_simple<float, true>(a, s) : launch_simple<float, false>(a, s);
}
hipError_t launch_prefill_simple_bf16(const PrefillArgs& a, hipStream_t s) {
  return a.cu_q ? launch_simple<bf16, true>(a, s) : launch_simple<bf16, false>(a, s);
}

}  // namespace gmla
