// Y = X W^T for bf16 X [M, K], W [N, K] (both contiguous along K), f32 accumulation,
// bf16 output: the dense projections of a Gated MLA layer ("Gated MLA", sections
// "Start from familiar attention" and "The channel-wise output gate": Q = X W_q^T,
// C = X W_c^T, K = C W_k^T, V = C W_v^T, G = X W_g^T, Y = O~ W_o^T).
//
// Design (gfx950):
//  * Tiles of X (BM rows) and W (BN rows) x 64 k move from global memory straight into
//    LDS with the LDS-direct form of the buffer load (no register staging), S stages
//    deep, so a stage is requested S-1 stages before it is used.  The buffer range of
//    a tile ends at the last valid row: rows past M (or N) load as zeros, with no
//    per-lane predicate.  Each stage is its own __shared__ array and the stage loop is
//    unrolled by S, so the compiler sees that a load into one stage does not alias the
//    reads of another (it would otherwise wait for every load before any LDS read).
//  * LDS rows are 128 bytes (64 k); the 16-byte chunk c of row r sits at chunk
//    c ^ ((r >> 1) & 7), which makes the fragment reads free of bank conflicts.
//  * The MFMA computes D = W X^T (v_mfma_f32_32x32x16_bf16, A = 32 rows of W, B = 32
//    rows of X): a lane then holds four consecutive output columns n of one output row
//    m per register quad; the tile is packed to bf16 in LDS and leaves as 16-byte
//    stores of whole 128-byte row segments.
//  * Workgroups are dealt so that the M blocks of one N block run on the same XCD:
//    the W tile they share is fetched from HBM once into that XCD's L2.
#include <type_traits>

#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int BK = 64;                 // k per stage: one 128-byte LDS row
constexpr int kBufferDword3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void_t;

// Hides a value from loop-invariant code motion, so address arithmetic derived from it
// is redone at each use (one VALU op) instead of occupying registers across the loop.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt vmcnt(N) (N < 64) leaving the other counters alone.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Barrier for the LDS stages: the caller has waited (vmcnt) for the loads the next
// stage reads; this waits for the wave's own LDS reads and meets the other waves.  A
// __syncthreads() would also wait for the loads meant to stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BM, int BN, int S, int WGM, int WGN>
struct Cfg {
  static constexpr int NW = WGM * WGN;          // waves
  static constexpr int NT = NW * 64;            // threads
  static constexpr int TM = BM / WGM;           // wave tile (rows of X)
  static constexpr int TN = BN / WGN;           // wave tile (rows of W)
  static constexpr int FM = TM / 32, FN = TN / 32;
  static constexpr int XL = BM / 8 / NW;        // 1 KB loads per wave per stage (X)
  static constexpr int WL = BN / 8 / NW;        // (W)
  static constexpr int LPS = XL + WL;           // loads per wave per stage
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(XL >= 1 && WL >= 1 && XL * NW * 8 == BM && WL * NW * 8 == BN, "load split");
  static_assert(S >= 2 && S <= 4, "stages");
};

// Stage buffers, one set per tile shape.  They live at namespace scope (not inside the
// kernel) so that each is a distinct LDS object to the compiler's alias analysis; a
// kernel is allocated only the buffers it references.
__shared__ __align__(16) bf16 wide_x0[256 * BK];
__shared__ __align__(16) bf16 wide_x1[256 * BK];
__shared__ __align__(16) bf16 wide_w0[192 * BK];
__shared__ __align__(16) bf16 wide_w1[192 * BK];
__shared__ __align__(16) bf16 deep_x0[256 * BK];
__shared__ __align__(16) bf16 deep_x1[256 * BK];
__shared__ __align__(16) bf16 deep_w0[384 * BK];
__shared__ __align__(16) bf16 deep_w1[384 * BK];
__shared__ __align__(16) bf16 split_x0[128 * BK];
__shared__ __align__(16) bf16 split_x1[128 * BK];
__shared__ __align__(16) bf16 split_w0[128 * BK];
__shared__ __align__(16) bf16 split_w1[128 * BK];
__shared__ __align__(16) bf16 narrow_x0[64 * BK];
__shared__ __align__(16) bf16 narrow_x1[64 * BK];
__shared__ __align__(16) bf16 narrow_x2[64 * BK];
__shared__ __align__(16) bf16 narrow_x3[64 * BK];
__shared__ __align__(16) bf16 narrow_w0[64 * BK];
__shared__ __align__(16) bf16 narrow_w1[64 * BK];
__shared__ __align__(16) bf16 narrow_w2[64 * BK];
__shared__ __align__(16) bf16 narrow_w3[64 * BK];

template <int BM, int BN, int S> struct StageSet;
template <> struct StageSet<256, 192, 2> {
  template <int B> static __device__ __forceinline__ bf16* x() { return B == 0 ? wide_x0 : wide_x1; }
  template <int B> static __device__ __forceinline__ bf16* w() { return B == 0 ? wide_w0 : wide_w1; }
};
template <> struct StageSet<256, 384, 2> {
  template <int B> static __device__ __forceinline__ bf16* x() { return B == 0 ? deep_x0 : deep_x1; }
  template <int B> static __device__ __forceinline__ bf16* w() { return B == 0 ? deep_w0 : deep_w1; }
};
template <> struct StageSet<128, 128, 2> {
  template <int B> static __device__ __forceinline__ bf16* x() { return B == 0 ? split_x0 : split_x1; }
  template <int B> static __device__ __forceinline__ bf16* w() { return B == 0 ? split_w0 : split_w1; }
};
template <> struct StageSet<64, 64, 4> {
  template <int B> static __device__ __forceinline__ bf16* x() {
    return B == 0 ? narrow_x0 : B == 1 ? narrow_x1 : B == 2 ? narrow_x2 : narrow_x3;
  }
  template <int B> static __device__ __forceinline__ bf16* w() {
    return B == 0 ? narrow_w0 : B == 1 ? narrow_w1 : B == 2 ? narrow_w2 : narrow_w3;
  }
};

template <int BM, int BN, int S, int WGM, int WGN, bool SPLIT = false>
__device__ __forceinline__ void gemm_lds_body(const GemmArgs& p, int nb1, int nmb, int total) {
  using C = Cfg<BM, BN, S, WGM, WGN>;
  auto xbuf = [&](auto b) __attribute__((always_inline)) -> bf16* {
    constexpr int B = decltype(b)::value;
    return StageSet<BM, BN, S>::template x<B>();
  };
  auto wbuf = [&](auto b) __attribute__((always_inline)) -> bf16* {
    constexpr int B = decltype(b)::value;
    return StageSet<BM, BN, S>::template w<B>();
  };

  // ---- workgroup -> (m block, n block); the m blocks of one n block share an XCD
  const int bid = blockIdx.x;
  const int per_xcd = total / kNumXcd;
  const int L = bid < per_xcd * kNumXcd ? (bid % kNumXcd) * per_xcd + bid / kNumXcd : bid;
  // split-K: L runs over the tiles of one range, then the next range, so an XCD takes
  // whole ranges (with eight ranges, one each) and reads its slab of X and W from the
  // last-level cache or HBM once for all its tiles, instead of every XCD reading
  // slabs of every range (2048 x 512 x 12288, 8 ranges: 571 -> 695 TFLOP/s with the
  // reduce, in alternating runs; the partials and their sum are bitwise the same)
  const int split = SPLIT ? L / (total / p.splits) : 0;
  const int tile = SPLIT ? L % (total / p.splits) : L;
  const int mb = tile % nmb;
  int nblk = tile / nmb;
  const bf16* W = (const bf16*)p.w;
  bf16* Y = (bf16*)p.y;
  int N = p.N;
  if (nblk >= nb1) {
    nblk -= nb1;
    W = (const bf16*)p.w2;
    Y = (bf16*)p.y2;
    N = p.N2;
  }
  const int M = p.M, K = p.K;
  const int m0 = mb * BM, n0 = nblk * BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wm = wave % WGM, wn = wave / WGM;

  // ---- buffer resources over this block's rows of X and W
  const int xrows = min(BM, M - m0), wrows = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.x + (int64_t)m0 * K), (short)0, xrows * K * 2, kBufferDword3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * K), (short)0, wrows * K * 2, kBufferDword3);

  // Load u of a wave fills 8 LDS rows (1 KB) in physical chunk order: lane i writes
  // row 8 (wave * L + u) + i / 8, physical chunk i mod 8, i.e. logical chunk
  // (i mod 8) ^ ((row >> 1) & 7) of that row; the stage's k offset is the scalar part.
  // The smaller tiles keep every load's offset in a register.  The 256 x 384 tile has
  // no room for ten (its accumulators take 192 of the wave's 256 registers) and keeps
  // two: with g = wave * L + u, bit 2 of the swizzle is g's parity, so the offset is
  // 16 g K (uniform) + lb0 or lb0 ^ 64 (per lane; K a multiple of 64 leaves bits 4..6
  // of the row term clear), one vector add per load.  Recomputing each offset from the
  // lane index took ~8 vector instructions per load (2048 x 12288 x 12288: 1332 ->
  // 1360 TFLOP/s in alternating runs, bitwise the same).
  constexpr bool kKeepOffsets = BN < 384;
  uint32_t xo[C::XL], wo[C::WL];
  auto offset = [&](int row, int ln) __attribute__((always_inline)) {
    return (uint32_t)(row * K * 2 + (((ln & 7) ^ ((row >> 1) & 7)) << 4));
  };
  if (kKeepOffsets) {
#pragma unroll
    for (int u = 0; u < C::XL; ++u) xo[u] = offset(8 * (wave * C::XL + u) + (lane >> 3), lane);
#pragma unroll
    for (int u = 0; u < C::WL; ++u) wo[u] = offset(8 * (wave * C::WL + u) + (lane >> 3), lane);
  }
  const uint32_t lb0 = (uint32_t)((lane >> 3) * K * 2 + (((lane & 7) ^ ((lane >> 4) & 3)) << 4));
  const uint32_t lb1 = lb0 ^ 64u;
  // offset of load u (group g) without a kept offset; the parity is u's when both
  // per-wave load counts are even.  The add is a volatile asm statement so that the
  // compiler neither hoists all ten sums out of the loop into registers the tile does
  // not have nor copies the base before each add (an empty asm barrier on the base
  // instead costs a move per load; 1384 -> 1392 TFLOP/s in alternating runs without
  // that move, bitwise the same).
  auto group_off = [&](int g, int u) __attribute__((always_inline)) {
    const bool odd = (C::XL % 2 == 0 && C::WL % 2 == 0) ? (u & 1) : (g & 1);
    uint32_t r;
    asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"((uint32_t)(g * 16 * K)), "v"(odd ? lb1 : lb0));
    return r;
  };
  const int kst0 = SPLIT ? split * p.kps : 0;  // first k stage of this range
  // load u of stage kt into buffer b (u < XL: rows of X, else rows of W)
  auto load_one = [&](int kt, auto b, int u) __attribute__((always_inline)) {
    const int koff = (kst0 + kt) * BK * 2;
    if (u < C::XL)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (lds_void_t*)(xbuf(b) + (wave * C::XL + u) * 512), 16,
          kKeepOffsets ? xo[u] : group_off(wave * C::XL + u, u), koff, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (lds_void_t*)(wbuf(b) + (wave * C::WL + (u - C::XL)) * 512), 16,
          kKeepOffsets ? wo[u - C::XL] : group_off(wave * C::WL + (u - C::XL), u - C::XL),
          koff, 0, 0);
  };
  auto load_stage = [&](int kt, auto b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::LPS; ++u) load_one(kt, b, u);
  };

  // Fragment reads: row l32 of a 32-row group, logical chunk 2 ks + hh, at byte
  // (frag_lane ^ 32 ks) from the group's first row (the swizzle only moves bits 4..6).
  const int frag_lane = l32 * 128 + ((hh ^ ((l32 >> 1) & 7)) << 4);

  f32x16 acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

  // One stage: 4 k-steps of 16; the fragments of k-step ks+1 are requested before the
  // MFMAs of k-step ks, so their LDS latency is covered (the fences keep that order).
  // On the 256 x 384 tiles the loads of the stage kt_next (>= 0) go out one after every
  // second MFMA from the first on: issued in one block after the barrier, their address
  // work (recomputed per stage on these tiles) and issue held back the first fragment
  // reads and MFMAs of every stage (2048 x 12288 x 12288: +6-7% in alternating runs,
  // bitwise the same result).  The other tiles keep the block: spread, the 512-deep
  // latent expansion ran 3% slower (its next stage arrives later) and the split-K
  // ranges the same.
  constexpr int kMfmaPerStage = (BK / 16) * C::FM * C::FN;
  constexpr bool kSpreadLoads = BM == 256 && BN == 384 && 2 * (C::LPS - 1) < kMfmaPerStage;
  auto compute = [&](auto b, int kt_next, auto bn) __attribute__((always_inline)) {
    const char* xt = (const char*)xbuf(b) + wm * C::TM * 128;
    const char* wt = (const char*)wbuf(b) + wn * C::TN * 128;
    const int fl = opaque(frag_lane);
    bf16x8 xf[2][C::FM], wf[2][C::FN];
    auto rd = [&](int ks, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < C::FM; ++j) xf[slot][j] = *(const bf16x8*)(xt + j * 4096 + (fl ^ (ks << 5)));
#pragma unroll
      for (int i = 0; i < C::FN; ++i) wf[slot][i] = *(const bf16x8*)(wt + i * 4096 + (fl ^ (ks << 5)));
    };
    rd(0, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) rd(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ks & 1][i], xf[ks & 1][j], acc[i][j], 0, 0, 0);
          if constexpr (kSpreadLoads) {
            const int m = (ks * C::FN + i) * C::FM + j;  // MFMA index in the stage
            if (kt_next >= 0 && m % 2 == 0 && m / 2 < C::LPS) {
              __builtin_amdgcn_sched_barrier(0);
              load_one(kt_next, bn, m / 2);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: stage kt is requested at iteration kt - (S - 1)
  const int nk = SPLIT ? min(p.kps, K / BK - kst0) : K / BK;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  load_stage(0, B0{});
  if (S > 2 && nk > 1) load_stage(1, B1{});
  if (S > 3 && nk > 2) load_stage(2, B2{});

  // iteration kt: wait for stage kt (the S-2 later stages may stay in flight), barrier
  // (every wave is done with stage kt-1, whose buffer the next request reuses),
  // request stage kt+S-1, compute stage kt.  This general form serves the last stages.
  auto step = [&](int kt, auto b) __attribute__((always_inline)) {
    constexpr int Bc = decltype(b)::value;
    const int ahead = min(nk - 1 - kt, S - 2);  // stages after kt already requested
    if (ahead >= 2)
      wait_vmcnt<2 * C::LPS>();
    else if (ahead == 1)
      wait_vmcnt<C::LPS>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    using Bn = std::integral_constant<int, (Bc + S - 1) % S>;
    const int kt_next = kt + S - 1 < nk ? kt + S - 1 : -1;
    if (!kSpreadLoads && kt_next >= 0) load_stage(kt_next, Bn{});
    compute(b, kSpreadLoads ? kt_next : -1, Bn{});
  };
  // main loop: every step has S-2 later stages in flight and requests one more
  auto step_full = [&](int kt, auto b) __attribute__((always_inline)) {
    constexpr int Bc = decltype(b)::value;
    wait_vmcnt<(S - 2) * C::LPS>();
    lds_barrier();
    using Bn = std::integral_constant<int, (Bc + S - 1) % S>;
    if (!kSpreadLoads) load_stage(kt + S - 1, Bn{});
    compute(b, kSpreadLoads ? kt + S - 1 : -1, Bn{});
  };
  int kt = 0;
  for (; kt + 2 * S - 2 < nk; kt += S) {
    step_full(kt, B0{});
    step_full(kt + 1, B1{});
    if (S > 2) step_full(kt + 2, B2{});
    if (S > 3) step_full(kt + 3, B3{});
  }
  // tail: at most 2 S - 2 stages, buffers continuing the rotation
  for (int r = 0; r < 2 * S - 2 && kt < nk; ++r, ++kt) {
    switch (kt % S) {
      case 0: step(kt, B0{}); break;
      case 1: step(kt, B1{}); break;
      case 2: if (S > 2) step(kt, B2{}); break;
      default: if (S > 3) step(kt, B3{}); break;
    }
  }

  // ---- epilogue: D[n][m] holds, in lane (m = l32), rows n = 8 (r/4) + 4 hh + r%4, i.e.
  // four consecutive n of one row m per register quad.  Stored as they are, each store
  // instruction would touch 32 rows with 16 bytes apiece; instead the tile goes through
  // LDS in chunks of 64 columns: every wave writes its part of the chunk into the first
  // X stage buffer (now idle; rows of 128 bytes, 16-byte unit q of row r at
  // q ^ ((r >> 1) & 7)), then the workgroup stores whole 128-byte row segments.
  if constexpr (SPLIT) {
    // float partials of this range: row m holds four consecutive columns per quad
    float* part = p.part + (int64_t)split * M * N;
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int m = m0 + wm * C::TM + j * 32 + l32;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = n0 + wn * C::TN + i * 32 + 8 * r4 + 4 * hh;
          f32x4 v;
          v[0] = acc[i][j][4 * r4]; v[1] = acc[i][j][4 * r4 + 1];
          v[2] = acc[i][j][4 * r4 + 2]; v[3] = acc[i][j][4 * r4 + 3];
          if (m < M && n < N) *(f32x4*)(part + (int64_t)m * N + n) = v;
        }
      }
    return;
  }
  static_assert(BN % 64 == 0, "64-column chunks");
  char* const stage = (char*)xbuf(B0{});  // BM rows x 64 bf16
#pragma unroll
  for (int c = 0; c < BN / 64; ++c) {
    lds_barrier();  // every wave is done with the stage buffer (main loop or last chunk)
#pragma unroll
    for (int i = 0; i < C::FN; ++i) {
      const int ncol = wn * C::TN + i * 32;  // first tile column of fragment i
      if (ncol < 64 * c || ncol >= 64 * c + 64) continue;  // uniform per wave
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int row = wm * C::TM + j * 32 + l32;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int col = ncol - 64 * c + 8 * r4 + 4 * hh;  // 0..63
          u32x2 v;
          v[0] = pack_bf16x2(acc[i][j][4 * r4 + 0], acc[i][j][4 * r4 + 1]);
          v[1] = pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
          *(u32x2*)(stage + row * 128 + (((col >> 3) ^ ((row >> 1) & 7)) << 4) + (col & 4) * 2) = v;
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < BM * 8 / C::NT; ++k) {
      const int piece = tid + k * C::NT;
      const int row = piece >> 3, q = piece & 7;
      const int m = m0 + row, n = n0 + 64 * c + 8 * q;
      const u32x4 v = *(const u32x4*)(stage + row * 128 + ((q ^ ((row >> 1) & 7)) << 4));
      if (m < M && n < N) *(u32x4*)(Y + (int64_t)m * N + n) = v;
    }
  }
}

// The kernels are plain (non-template) functions around the templated body: the host
// pass then never instantiates device-only builtins.
__global__ __launch_bounds__(512, 1) void gemm_lds_wide_kernel(GemmArgs p, int nb1, int nmb,
                                                               int total) {
  gemm_lds_body<256, 192, 2, 4, 2>(p, nb1, nmb, total);
}
__global__ __launch_bounds__(512, 1) void gemm_lds_deep_kernel(GemmArgs p, int nb1, int nmb,
                                                               int total) {
  gemm_lds_body<256, 384, 2, 2, 4>(p, nb1, nmb, total);
}
__global__ __launch_bounds__(256, 2) void gemm_lds_narrow_kernel(GemmArgs p, int nb1, int nmb,
                                                                 int total) {
  gemm_lds_body<64, 64, 4, 2, 2>(p, nb1, nmb, total);
}

// Split-K ranges of few, deep output tiles: 128 x 128 tiles, 4 waves of 64 x 64, two
// 64-deep stages (64 KB of LDS, two workgroups per CU); float partials, summed below.
__global__ __launch_bounds__(256, 2) void gemm_lds_splitk_kernel(GemmArgs p, int nb1, int nmb,
                                                                 int total) {
  gemm_lds_body<128, 128, 2, 2, 2, true>(p, nb1, nmb, total);
}

// Y[m][n] = bf16(sum over ranges of part[r][m][n]), four columns per thread.
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(const float* part, int splits,
                                                                 int64_t mn4, int64_t mn,
                                                                 bf16* y) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < mn4; i += (int64_t)gridDim.x * 256) {
    f32x4 acc = *(const f32x4*)(part + 4 * i);
    for (int r = 1; r < splits; ++r) {
      const f32x4 v = *(const f32x4*)(part + (int64_t)r * mn + 4 * i);
      acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
    }
    u32x2 w;
    w[0] = pack_bf16x2(acc[0], acc[1]);
    w[1] = pack_bf16x2(acc[2], acc[3]);
    *(u32x2*)(y + 4 * i) = w;
  }
}

template <int BM, int BN, int NT>
hipError_t launch_cfg(void (*kernel)(GemmArgs, int, int, int), const GemmArgs& p,
                      hipStream_t s) {
  const int nmb = (p.M + BM - 1) / BM;
  const int nb1 = (p.N + BN - 1) / BN;
  const int nb2 = p.w2 ? (p.N2 + BN - 1) / BN : 0;
  const long total = (long)nmb * (nb1 + nb2);
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(NT), 0, s, p, nb1, nmb, (int)total);
  return hipGetLastError();
}

}  // namespace

bool gemm_lds_supported(const GemmArgs& p) {
  const auto al = [](const void* q, uintptr_t a) { return ((uintptr_t)q % a) == 0; };
  if (p.g || p.K % BK || p.N % 8 || (p.w2 && p.N2 % 8)) return false;
  if (!al(p.x, 16) || !al(p.w, 16) || !al(p.y, 16) || (p.w2 && (!al(p.w2, 16) || !al(p.y2, 16))))
    return false;
  // byte offsets inside one block's rows are 32-bit
  return (int64_t)256 * p.K * 2 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_lds(const GemmArgs& p, hipStream_t s) {
  // Deep products (K >= 512) with enough 256 x 384 tiles to fill the CUs: 8 waves of
  // 128 x 96, 2 stages (160 KB of LDS, one workgroup per CU); per flop they move 29% fewer
  // tile bytes global -> LDS and read 30% fewer fragment bytes than 256 x 192 tiles
  // (measured on 2048 x 12288 x 12288: 1076 -> 1243 TFLOP/s).  With the tile loads issued
  // among the MFMAs they also win at K = 512, the latent expansion (2048 x 24576 x 512:
  // 846 -> 908 TFLOP/s in alternating runs; before that change they lost there, 775 ->
  // 701).
  // Wide outputs: 256 x 192 tiles, 8 waves of 64 x 96, 2 stages (112 KB of LDS, one
  // workgroup per CU); measured against 256 x 128 tiles with 3 stages: 5% faster on the
  // 12288-deep projections, 16% on the 512-deep latent expansion.  Narrow outputs (too
  // few wide tiles to fill 256 CUs): 64 x 64 tiles, 4 waves of 32 x 32, 4 stages (64 KB,
  // two workgroups per CU).
  const long deep = (long)((p.M + 255) / 256) *
                    ((p.N + 383) / 384 + (p.w2 ? (p.N2 + 383) / 384 : 0));
  if (deep >= 256 && p.K >= 512 && p.N % 384 == 0 && (!p.w2 || p.N2 % 384 == 0) &&
      (int64_t)384 * p.K * 2 < ((int64_t)1 << 31))
    return launch_cfg<256, 384, 512>(gemm_lds_deep_kernel, p, s);
  const long big = (long)((p.M + 255) / 256) *
                   ((p.N + 191) / 192 + (p.w2 ? (p.N2 + 191) / 192 : 0));
  if (big >= 512) return launch_cfg<256, 192, 512>(gemm_lds_wide_kernel, p, s);
  return launch_cfg<64, 64, 256>(gemm_lds_narrow_kernel, p, s);
}

void gemm_splitk_plan(int M, int N, int K, int* splits, int* kps) {
  *splits = 1;
  *kps = K / BK;
  if (M <= 0 || N <= 0 || K % BK || N % 8) return;
  const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
  const int nk = K / BK;
  // only products whose output alone cannot fill the 256 CUs twice, and at least eight
  // 64-deep stages per range
  if (tiles >= 256 || nk < 16) return;
  long s = (512 + tiles - 1) / tiles;
  if (s > nk / 8) s = nk / 8;
  if (s < 2) return;
  const int k = (int)((nk + s - 1) / s);
  *kps = k;
  *splits = (nk + k - 1) / k;
}

hipError_t launch_gemm_splitk(const GemmArgs& p, hipStream_t s) {
  const int nmb = (p.M + 127) / 128;
  const int nb1 = (p.N + 127) / 128;
  const long total = (long)nmb * nb1 * p.splits;
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_lds_splitk_kernel, dim3((unsigned)total), dim3(256), 0, s, p, nb1, nmb,
                     (int)total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mn = (int64_t)p.M * p.N;
  int64_t blocks = (mn / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gemm_splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p.part,
                     p.splits, mn / 4, mn, (bf16*)p.y);
  return hipGetLastError();
}

}  // namespace gmla
