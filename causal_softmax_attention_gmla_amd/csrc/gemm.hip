// Y = A W^T on the matrix cores: the projections of a Gated MLA layer ("Gated MLA":
// Q = X W_q^T, C = X W_c^T, K = C W_k^T, V = C W_v^T, G = X W_g^T, and the output
// projection [sigmoid(G) (.) O~] W_o^T, sections "Start from familiar attention" and
// "The channel-wise output gate").  Weights are stored [out, in], so both operands
// are contiguous along the reduction axis and every MFMA fragment is one 16-byte
// LDS read.
//
// Options folded into the same kernel:
//  * a gate prologue: when gate logits G [M, K] are given, the A operand is
//    sigmoid(G) * A, formed while the A tile is staged (gate BEFORE the projection);
//  * a second weight/output pair: columns [N, N + N2) of the grid use W2 and write Y2,
//    so K and V come out of one launch over the latent C.
//
// bf16: workgroup tile 128 x 128 x 64, 4 waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16
// tiles), tiles double-buffered in LDS with the next tile's global loads in flight
// during the MFMAs.  f32: a plain LDS-tiled FMA kernel (exact float32 products).
#include "gmla_internal.h"

namespace gmla {
namespace {

// ------------------------------------------------------------------ bf16 MFMA
constexpr int GBM = 128, GBN = 128, GBK = 64;
constexpr int GLD = GBK + 8;  // LDS row stride (bf16): 144 B, conflict-free fragment reads
constexpr int GNT = 256;

struct __align__(16) GemmSmem {
  bf16 a[2][GBM * GLD];
  bf16 b[2][GBN * GLD];
};

__device__ __forceinline__ uint32_t gate_pair(uint32_t x, uint32_t g) {
  const float lo = bf16_lo(x) * sigmoidf_(bf16_lo(g));
  const float hi = bf16_hi(x) * sigmoidf_(bf16_hi(g));
  return pack_bf16x2(lo, hi);
}

__global__ __launch_bounds__(GNT, 2) void gemm_bf16_kernel(GemmArgs p, int nb1) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  // column block: the first nb1 blocks use (w, y, N), the rest (w2, y2, N2)
  int nblk = blockIdx.y;
  const bf16* W = (const bf16*)p.w;
  bf16* Y = (bf16*)p.y;
  int N = p.N;
  if (nblk >= nb1) {
    nblk -= nb1;
    W = (const bf16*)p.w2;
    Y = (bf16*)p.y2;
    N = p.N2;
  }
  const int m0 = blockIdx.x * GBM, n0 = nblk * GBN;
  const int M = p.M, K = p.K;
  const bf16* X = (const bf16*)p.x;
  const bf16* G = (const bf16*)p.g;

  u32x4 areg[4], breg[4], greg[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = i * GNT + tid;
      const int r = id >> 3, c = (id & 7) * 8;
      const int k = k0 + c;
      const int m = m0 + r, n = n0 + r;
      const bool ka = k < K;
      areg[i] = (m < M && ka) ? *(const u32x4*)(X + (int64_t)m * K + k) : u32x4{};
      if (G) greg[i] = (m < M && ka) ? *(const u32x4*)(G + (int64_t)m * K + k) : u32x4{};
      breg[i] = (n < N && ka) ? *(const u32x4*)(W + (int64_t)n * K + k) : u32x4{};
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = i * GNT + tid;
      const int r = id >> 3, c = (id & 7) * 8;
      u32x4 av = areg[i];
      if (G) {
#pragma unroll
        for (int w = 0; w < 4; ++w) av[w] = gate_pair(av[w], greg[i][w]);
      }
      *(u32x4*)(&sm.a[buf][r * GLD + c]) = av;
      *(u32x4*)(&sm.b[buf][r * GLD + c]) = breg[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (K + GBK - 1) / GBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *(const bf16x8*)(&sm.a[buf][(wm * 64 + i * 32 + l32) * GLD + ks * 16 + hh * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *(const bf16x8*)(&sm.b[buf][(wn * 64 + j * 32 + l32) * GLD + ks * 16 + hh * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // D[m][n]: lane holds column n = l32 and rows 8*(r/4) + 4*hh + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (m < M) Y[(int64_t)m * N + n] = f32_to_bf16(acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------------ f32 FMA
constexpr int FT = 64, FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs p, int nb1) {
  __shared__ float as[FK][FT + 1];
  __shared__ float bs[FK][FT + 1];
  int nblk = blockIdx.y;
  const float* W = (const float*)p.w;
  float* Y = (float*)p.y;
  int N = p.N;
  if (nblk >= nb1) {
    nblk -= nb1;
    W = (const float*)p.w2;
    Y = (float*)p.y2;
    N = p.N2;
  }
  const int m0 = blockIdx.x * FT, n0 = nblk * FT;
  const int M = p.M, K = p.K;
  const float* X = (const float*)p.x;
  const float* G = (const float*)p.g;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int idx = tid; idx < FT * FK; idx += 256) {
      const int r = idx / FK, c = idx % FK;
      const int k = k0 + c;
      float av = 0.0f, bv = 0.0f;
      if (m0 + r < M && k < K) {
        av = X[(int64_t)(m0 + r) * K + k];
        if (G) av *= 1.0f / (1.0f + expf(-G[(int64_t)(m0 + r) * K + k]));
      }
      if (n0 + r < N && k < K) bv = W[(int64_t)(n0 + r) * K + k];
      as[c][r] = av;
      bs[c][r] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < FK; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_fmaf(as[c][ty * 4 + i], bs[c][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) Y[(int64_t)m * N + n] = acc[i][j];
    }
}

// ------------------------------------------------------------------ gate only
template <typename T>
__global__ __launch_bounds__(256) void gate_kernel(int64_t n, const T* g, const T* x, T* y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float v = Elem<T>::load(x + i);
    if (g) v *= sigmoidf_(Elem<T>::load(g + i));
    Elem<T>::store(y + i, v);
  }
}

// bf16, 8 elements per lane with 16-byte loads and stores (same arithmetic per element
// as gate_kernel, so the two agree bit for bit)
__global__ __launch_bounds__(256) void gate_bf16x8_kernel(int64_t n8, const bf16* g, const bf16* x,
                                                          bf16* y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 xv = *(const u32x4*)(x + 8 * i);
    const u32x4 gv = *(const u32x4*)(g + 8 * i);
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = gate_pair(xv[j], gv[j]);
    *(u32x4*)(y + 8 * i) = out;
  }
}

}  // namespace

hipError_t launch_gemm(int dtype, const GemmArgs& p, hipStream_t s) {
  if (dtype == 1 && gemm_lds_supported(p)) return launch_gemm_lds(p, s);
  if (dtype == 1) {
    const int nb1 = (p.N + GBN - 1) / GBN;
    const int nb2 = p.w2 ? (p.N2 + GBN - 1) / GBN : 0;
    hipLaunchKernelGGL(gemm_bf16_kernel, dim3((p.M + GBM - 1) / GBM, nb1 + nb2), dim3(GNT), 0, s,
                       p, nb1);
  } else {
    const int nb1 = (p.N + FT - 1) / FT;
    const int nb2 = p.w2 ? (p.N2 + FT - 1) / FT : 0;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((p.M + FT - 1) / FT, nb1 + nb2), dim3(256), 0, s, p,
                       nb1);
  }
  return hipGetLastError();
}

hipError_t launch_gate_only(int dtype, int64_t n, const void* g, const void* x, void* y,
                            hipStream_t s) {
  const auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  if (dtype == 1 && g && n % 8 == 0 && al16(g) && al16(x) && al16(y)) {
    int64_t blocks = (n / 8 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gate_bf16x8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n / 8,
                       (const bf16*)g, (const bf16*)x, (bf16*)y);
    return hipGetLastError();
  }
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (dtype == 1)
    hipLaunchKernelGGL(gate_kernel<bf16>, dim3((unsigned)blocks), dim3(256), 0, s, n,
                       (const bf16*)g, (const bf16*)x, (bf16*)y);
  else
    hipLaunchKernelGGL(gate_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, n,
                       (const float*)g, (const float*)x, (float*)y);
  return hipGetLastError();
}

}  // namespace gmla
