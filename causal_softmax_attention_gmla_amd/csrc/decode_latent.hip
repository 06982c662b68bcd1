// Decode over the latent cache: one new query per (batch, head) against N cached tokens
// whose keys and values exist only as the latent rows c_n of width d_c ("Gated MLA",
// section "Start from familiar attention": K = C W_k^T, V = C W_v^T, and "Common mistakes
// to avoid": the cache is the compact latent tensor, not reconstructed keys and values;
// "Le Transformer et l'attention", "MLA - compresser en un vecteur latent": 512 cached
// values per token against 96 x 256 for full keys and values).  The query sits at
// position N - 1 and sees every cached token ("Kimi K3 - Softmax over keys").
//
// The keys and values are never formed.  With W_k,h and W_v,h the 128 rows of W_k and
// W_v that belong to head h, the products regroup exactly:
//     s_n = scale * q_h . (W_k,h c_n) = (scale * W_k,h^T q_h) . c_n = q'_h . c_n
//     o_h = sum_n p_n (W_v,h c_n)     = W_v,h (sum_n p_n c_n)      = W_v,h u_h
// so every head attends directly over the shared latent rows, and the per-token bytes
// read are the d_c latent values (shared by all heads) instead of H * 256 key and value
// values.  Three launches:
//  1. absorb:  q'[b, h, :] = scale * log2(e) * W_k,h^T q[b, h, :]  (bf16, workspace);
//  2. split:   one workgroup per (key range, 32-head block, batch row), the head blocks
//     of a (range, row) pair on one XCD.  The workgroup's key range is walked
//     in tiles of 32 latent rows staged in LDS (buffer loads in the LDS-direct form, three
//     tiles ahead; rows past N load as zeros).  Wave w owns latent channels
//     [w d_c / 4, (w + 1) d_c / 4): it forms its share of the scores S^T = C q'^T
//     (v_mfma_f32_32x32x16_bf16, keys x heads), the four shares are summed through LDS in
//     a fixed order (every wave then holds the same scores), the online softmax runs in
//     base 2 per head, and the wave accumulates its channels of U^T = C^T P^T, reading
//     the tile transposed with ds_read_b64_tr_b16 so that the weights never move between
//     lanes.  Each split writes (m, l, u[d_c]) per head.
//  3. merge:   per (head, 32 output channels), for every batch row: the log-sum-exp merge
//     of the splits (an exact regrouping of the one softmax), u / l, then
//     o = W_v,h u, the optional sigmoid gate ("Gated MLA", section "The channel-wise
//     output gate"), and the bf16 store into [B, H*128].
#include <type_traits>

#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int LHD = 128;          // head width
constexpr int HB = 32;            // heads per split workgroup
constexpr int KT = 32;            // latent rows per tile
constexpr int NT = 256;           // 4 waves
constexpr int kMaxDc = 512;
constexpr float kLazyRescale = 8.0f;  // raise the running max only past 2^8 growth
constexpr int kBufferDword3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// One array per buffer, so the compiler can tell a load into one from reads of another.
// Four tile buffers: tile j + 3 is requested while tile j is used, so three tiles' loads
// (96 KB at d_c = 512) are in flight per workgroup while it computes: a step then waits for
// a third of the memory latency rather than half.
__shared__ __align__(16) bf16 lat_c0[KT * kMaxDc];
__shared__ __align__(16) bf16 lat_c1[KT * kMaxDc];
__shared__ __align__(16) bf16 lat_c2[KT * kMaxDc];
__shared__ __align__(16) bf16 lat_c3[KT * kMaxDc];
// score shares [wave][quad][lane]: written after a tile's first barrier and read after its
// second, so the next tile's first barrier already separates the reads from the rewrite
__shared__ __align__(16) f32x4 lat_x[4 * 4 * 64];
template <int P> __device__ __forceinline__ bf16* cbuf() {
  return P == 0 ? lat_c0 : P == 1 ? lat_c1 : P == 2 ? lat_c2 : lat_c3;
}

// s_waitcnt vmcnt(N) (N < 64) leaving the other counters alone.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Workgroup barrier for LDS data: waits for this wave's LDS operations only, so tile loads
// meant to stay in flight are not waited for (a __syncthreads() would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Swizzle of the 16-byte chunk index inside each group of 16 chunks of a tile row.  The
// score reads take one chunk of 32 consecutive rows; the transposing reads take four
// chunks of rows 4i .. 4i+3: rows 0..3 XOR bits 2-3 and consecutive rows differ in the
// low bits, so both kinds spread over distinct banks.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int phys_chunk(int row, int c) { return (c & ~15) | ((c & 15) ^ swz(row)); }

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// ---------------------------------------------------------------- 1. absorb W_k into q
// grid (d_c / 64, H); thread t: latent channel c = 64 blockIdx.x + t mod 64 and head
// channels [32 (t / 64), 32 (t / 64) + 32) of W_k (its 32 values stay in registers).  The
// queries of head h for up to 32 batch rows at a time are staged in LDS; every thread
// forms its partial dot products for all of them, and one barrier later the four
// partials of each (row, c) are summed.  No global load waits inside the row loop.
constexpr int kAbsorbRows = 32;
template <int DC>
__global__ __launch_bounds__(NT) void latent_absorb_kernel(LatentDecodeArgs a) {
  __shared__ __align__(16) float qs[kAbsorbRows][LHD];
  __shared__ float red[4][kAbsorbRows][64];
  const int tid = threadIdx.x, lane = tid & 63, dg = tid >> 6;
  const int h = blockIdx.y;
  const int c = blockIdx.x * 64 + lane;
  const bf16* wk = a.wk + ((int64_t)h * LHD + dg * 32) * DC + c;
  float w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = bf16_to_f32(wk[(int64_t)i * DC]);
  for (int b0 = 0; b0 < a.B; b0 += kAbsorbRows) {
    const int nb = min(kAbsorbRows, a.B - b0);
    __syncthreads();  // qs and red are free again
    // rows b0 .. b0+nb-1 of q[:, h, :]: 16 pieces of 8 values per row
    for (int piece = tid; piece < nb * 16; piece += NT) {
      const int r = piece >> 4, k = piece & 15;
      const u32x4 v = *(const u32x4*)(a.q + ((int64_t)(b0 + r) * a.H + h) * LHD + 8 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[r][8 * k + 2 * e] = bf16_lo(v[e]);
        qs[r][8 * k + 2 * e + 1] = bf16_hi(v[e]);
      }
    }
    __syncthreads();
    for (int r = 0; r < nb; ++r) {
      float acc = 0.0f;
#pragma unroll
      for (int i4 = 0; i4 < 8; ++i4) {
        const f32x4 qv = *(const f32x4*)&qs[r][dg * 32 + 4 * i4];
        acc = __builtin_fmaf(qv[0], w[4 * i4], acc);
        acc = __builtin_fmaf(qv[1], w[4 * i4 + 1], acc);
        acc = __builtin_fmaf(qv[2], w[4 * i4 + 2], acc);
        acc = __builtin_fmaf(qv[3], w[4 * i4 + 3], acc);
      }
      red[dg][r][lane] = acc;
    }
    __syncthreads();
    for (int o = tid; o < nb * 64; o += NT) {
      const int r = o >> 6, l = o & 63;
      const float sum = ((red[0][r][l] + red[1][r][l]) + red[2][r][l]) + red[3][r][l];
      a.qp[((int64_t)(b0 + r) * a.H + h) * DC + blockIdx.x * 64 + l] = f32_to_bf16(sum * a.c2);
    }
  }
}

// ---------------------------------------------------------------- 2. split attention
template <int DC>
__device__ __forceinline__ void latent_split_body(const LatentDecodeArgs& a) {
  constexpr int WDC = DC / 4;      // latent channels of one wave
  constexpr int KS = WDC / 16;     // k-steps of the score MFMA
  constexpr int DB = WDC / 32;     // 32-channel blocks of U^T
  constexpr int RCH = DC / 8;      // 16-byte chunks per tile row
  constexpr int RPI = 64 / RCH;    // tile rows per 1 KB load instruction
  constexpr int LPW = KT / RPI / 4;  // load instructions per wave per tile
  static_assert(DC % 128 == 0 && DC <= kMaxDc, "latent width");

  // Grid (8 nhb, npy, npz): workgroup (x + 8 hb, g) takes head block hb of range pair
  // p = 8 g + x, i.e. (split p mod splits, batch row p / splits).  Workgroups are dealt to
  // the XCDs round-robin in launch order, so the nhb head blocks of one pair run on the
  // same XCD and read its latent rows through the same L2.
  const int hb = blockIdx.x >> 3;
  const int pair = 8 * (blockIdx.y + gridDim.y * blockIdx.z) + (blockIdx.x & 7);
  if (pair >= a.splits * a.B) return;
  const int split = pair % a.splits, b = pair / a.splits;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int head = hb * HB + l32;
  const bool hvalid = head < a.H;
  // rows cached for this batch row: all N, or its own length (a range past it is empty
  // and leaves m = -inf, l = 0, which the merge weighs 0)
  const int Nb = a.lens ? min(max(a.lens[b], 0), a.N) : a.N;
  const int n0 = split * a.kps;
  // (the ranges' ends, rounded up to whole tiles, can pass 2^31 for N near the key limit)
  const int n1 = (int)min((int64_t)Nb, (int64_t)n0 + a.kps);
  const int wd0 = wave * WDC;
  const bf16* Cb = a.c + (int64_t)b * a.csb;
  const int64_t csn = a.csn;

  // q' fragments (B operand of S^T = C q'^T): head l32, channels wd0 + 16 ks + 8 hh .. +8
  bf16x8 qf[KS];
  {
    const bf16* qrow = a.qp + ((int64_t)b * a.H + (hvalid ? head : 0)) * DC + wd0 + hh * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = hvalid ? *(const bf16x8*)(qrow + ks * 16) : bf16x8{};
  }

  // Tile loads: instruction u of wave w fills LDS bytes [1 KB (w LPW + u), +1 KB), i.e.
  // rows RPI (w LPW + u) .. +RPI-1; lane i writes physical chunk i mod RCH of row
  // i / RCH, fetching the logical chunk that the swizzle puts there.
  uint32_t loff[LPW];
#pragma unroll
  for (int u = 0; u < LPW; ++u) {
    const int row = RPI * (wave * LPW + u) + lane / RCH;
    const int pc = lane % RCH;
    const int lc = (pc & ~15) | ((pc & 15) ^ swz(row));
    loff[u] = (uint32_t)(row * csn * 2 + lc * 16);
  }
  auto load_tile = [&](int tile, auto buf) __attribute__((always_inline)) {
    const int r0 = tile * KT;
    const int rows = min(KT, Nb - r0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Cb + (int64_t)r0 * csn), (short)0, (int)((int64_t)(rows - 1) * csn * 2 + DC * 2),
        kBufferDword3);
#pragma unroll
    for (int u = 0; u < LPW; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_void_t*)(cbuf<decltype(buf)::value>() + (wave * LPW + u) * 512), 16, loff[u], 0,
          0, 0);
  };

  // score fragment (A operand): row l32, logical chunk wd0/8 + 2 ks + hh
  auto sread = [&](const bf16* t, int ks) __attribute__((always_inline)) -> bf16x8 {
    const int lc = wd0 / 8 + 2 * ks + hh;
    return *(const bf16x8*)(t + l32 * DC + phys_chunk(l32, lc) * 8);
  };
  // transposed fragment of U^T = C^T P^T (A operand): lane p of each 16-lane group points
  // at row 16 kk + 4 hh + p/4 (and that + 8), channels dbase + 4 (p mod 4) .. +3 with
  // dbase = wd0 + 32 dblk + 16 ((lane / 16) mod 2); the transposing read hands lane p the
  // channel dbase + p of those four rows: rows 16 kk + 4 hh + {0..3, 8..11} of channel
  // wd0 + 32 dblk + (lane mod 32), the keys of this lane's P^T registers.
  const int p16 = lane & 15;
  auto tread = [&](const bf16* t, int kk, int dblk) __attribute__((always_inline)) -> bf16x8 {
    const int row = 16 * kk + 4 * hh + (p16 >> 2);
    const int d0 = wd0 + 32 * dblk + 16 * ((lane >> 4) & 1) + 4 * (p16 & 3);
    const bf16* lo = t + row * DC + phys_chunk(row, d0 >> 3) * 8 + (d0 & 7);
    const bf16* hi = t + (row + 8) * DC + phys_chunk(row + 8, d0 >> 3) * 8 + (d0 & 7);
    const v4i16 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)lo);
    const v4i16 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)hi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 uacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) uacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max, base-2 units (q' carries scale * log2 e)
  float l_run = 0.0f;       // this lane half's sum of bf16-rounded weights
  bf16x2 ones2;
  ones2[0] = (bf16)1.0f;
  ones2[1] = (bf16)1.0f;

  const int t_first = n0 / KT;
  const int t_last = (n1 + KT - 1) / KT;  // exclusive; splits start on tile boundaries

  auto step = [&](int tile, auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    // this wave's loads of the tile are done when at most the next two tiles' are in flight
    if (tile + 2 < t_last)
      wait_vmcnt<2 * LPW>();
    else if (tile + 1 < t_last)
      wait_vmcnt<LPW>();
    else
      wait_vmcnt<0>();
    lds_barrier();  // tile in LDS; every wave is done with tile - 1 (whose buffer is refilled)
    if (tile + 3 < t_last) load_tile(tile + 3, std::integral_constant<int, (P + 3) % 4>{});
    const bf16* t = cbuf<P>();
    // this wave's share of the scores, over its latent channels
    f32x16 sp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sread(t, ks), qf[ks], sp, 0, 0, 0);
    f32x4* xs = lat_x;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v;
      v[0] = sp[4 * q4]; v[1] = sp[4 * q4 + 1]; v[2] = sp[4 * q4 + 2]; v[3] = sp[4 * q4 + 3];
      xs[(wave * 4 + q4) * 64 + lane] = v;
    }
    lds_barrier();
    // the whole scores, summed over the four shares in the same order in every wave
    f32x16 s;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 v = xs[q4 * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 x = xs[(w * 4 + q4) * 64 + lane];
        v[0] += x[0]; v[1] += x[1]; v[2] += x[2]; v[3] += x[3];
      }
      s[4 * q4] = v[0]; s[4 * q4 + 1] = v[1]; s[4 * q4 + 2] = v[2]; s[4 * q4 + 3] = v[3];
    }
    // rows past the cache end score -inf (zeros were loaded there)
    if (tile * KT + KT > Nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = tile * KT + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key >= Nb) s[r] = -INFINITY;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    mt = swap_halves_max(mt);
    const bool grow = mt > m_run + kLazyRescale;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mt) : 1.0f;  // m_run = -inf: 0
      m_run = grow ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) uacc[i][r] *= alpha;
    }
    // weights, rounded to bf16: the B operand of U^T = C^T P^T for k-steps 0 and 1
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      bf16x2 pp;
      pp[0] = (bf16)fast_exp2(s[r] - m_run);
      pp[1] = (bf16)fast_exp2(s[r + 1] - m_run);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, l_run, false);
      pb[r >> 3][r & 7] = pp[0];
      pb[r >> 3][(r & 7) + 1] = pp[1];
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dblk = 0; dblk < DB; ++dblk)
        uacc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tread(t, kk, dblk), pb[kk], uacc[dblk],
                                                             0, 0, 0);
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  if (t_first < t_last) load_tile(t_first, B0{});
  if (t_first + 1 < t_last) load_tile(t_first + 1, B1{});
  if (t_first + 2 < t_last) load_tile(t_first + 2, B2{});
  int tile = t_first;
  for (; tile + 3 < t_last; tile += 4) {
    step(tile, B0{});
    step(tile + 1, B1{});
    step(tile + 2, B2{});
    step(tile + 3, B3{});
  }
  if (tile < t_last) step(tile, B0{});
  if (tile + 1 < t_last) step(tile + 1, B1{});
  if (tile + 2 < t_last) step(tile + 2, B2{});

  // ---- partials of this split: (m, l) per head, and this wave's channels of u
  const float l_tot = swap_halves_sum(l_run);
  if (!hvalid) return;
  const int64_t slot = ((int64_t)b * a.H + head) * a.splits + split;
  if (wave == 0 && hh == 0) {
    a.ml[2 * slot] = m_run;
    a.ml[2 * slot + 1] = l_tot;
  }
  float* urow = a.u + slot * DC;
#pragma unroll
  for (int dblk = 0; dblk < DB; ++dblk)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 v;
      v[0] = uacc[dblk][4 * r4]; v[1] = uacc[dblk][4 * r4 + 1];
      v[2] = uacc[dblk][4 * r4 + 2]; v[3] = uacc[dblk][4 * r4 + 3];
      *(f32x4*)(urow + wd0 + 32 * dblk + 8 * r4 + 4 * hh) = v;
    }
}

// ---------------------------------------------------------------- 3. merge, W_v, gate
// One workgroup per (head, 32 output channels, kMergeRows batch rows), all of a head's on
// one XCD; thread t: output channel d = d0 + t / 8; part
// p = t mod 8 takes latent channels 64 i + 8 p .. +7 (i = 0 .. DC/64 - 1) of the W_v row.
// For its batch rows the workgroup first turns each row's split maxima into merge weights
// f_j = 2^(m_j - m) and 1 / l in LDS (one wave per row), then merges u for all its rows
// with independent loads, and finally multiplies by W_v.
constexpr int kMergeRows = 2;
constexpr int kMaxMergeSplits = 1024;
template <int DC>
__global__ __launch_bounds__(NT) void latent_merge_kernel(LatentDecodeArgs a) {
  constexpr int NI = DC / 64;
  __shared__ __align__(16) float us[kMergeRows][DC];
  __shared__ float fw[kMergeRows][kMaxMergeSplits];
  __shared__ float inv_l[kMergeRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Grid (8 G, ceil(H / 8)) with G = 4 ceil(B / kMergeRows) workgroups per head: workgroup
  // (x + 8 r, y) takes head 8 y + x, channel block r mod 4 and the batch rows of block r / 4.
  // Dealt to the XCDs round-robin in launch order, all G workgroups of a head run on one
  // XCD, so its W_v rows and split partials are read from HBM once and then from L2.
  const int slot = blockIdx.x >> 3;
  const int h = 8 * blockIdx.y + (blockIdx.x & 7);
  if (h >= a.H) return;
  const int cb = slot & 3;
  const int b0 = (slot >> 2) * kMergeRows;
  const int nb = min(kMergeRows, a.B - b0);
  const int S = a.splits;
  // this thread's W_v values (issued first: their latency overlaps the merge)
  const int d = cb * 32 + (tid >> 3);
  const int p = tid & 7;
  u32x4 wv[NI];
  {
    const bf16* wrow = a.wv + ((int64_t)h * LHD + d) * DC + 8 * p;
#pragma unroll
    for (int i = 0; i < NI; ++i) wv[i] = *(const u32x4*)(wrow + 64 * i);
  }
  // merge weights: wave r takes batch row b0 + r
  if (wave < nb) {
    const float* ml = a.ml + 2 * (((int64_t)(b0 + wave) * a.H + h) * S);
    float m = -INFINITY;
    for (int j = lane; j < S; j += 64) m = fmaxf(m, ml[2 * j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.0f;
    for (int j = lane; j < S; j += 64) {
      const float mj = ml[2 * j];
      // a range with no key (never produced) gets weight 0
      const float f = mj == -INFINITY ? 0.0f : fast_exp2(mj - m);
      fw[wave][j] = f;
      l = __builtin_fmaf(ml[2 * j + 1], f, l);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    // (a row with no cached token, possible only with per-row lengths, has l = 0 and
    // gets zeros)
    if (lane == 0) inv_l[wave] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  __syncthreads();
  // merged, normalised u of every row; thread t takes channels t + NT e.  Rows past the
  // batch end read row 0 with weight 0, so the loads carry no branch and the unrolled
  // loop keeps all of them in flight.
  constexpr int CPT = DC >= NT ? DC / NT : 1;
  const bool cvalid = DC >= NT || tid < DC;
  const int ct = cvalid ? tid : 0;
  float acc[kMergeRows][CPT];
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r)
#pragma unroll
    for (int e = 0; e < CPT; ++e) acc[r][e] = 0.0f;
  const float* ubase[kMergeRows];
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r)
    ubase[r] = a.u + (((int64_t)(b0 + (r < nb ? r : 0)) * a.H + h) * S) * DC + ct;
#pragma unroll 4
  for (int j = 0; j < S; ++j) {
#pragma unroll
    for (int r = 0; r < kMergeRows; ++r) {
      const float f = r < nb ? fw[r][j] : 0.0f;
#pragma unroll
      for (int e = 0; e < CPT; ++e)
        acc[r][e] = __builtin_fmaf(ubase[r][(int64_t)j * DC + NT * e], f, acc[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < kMergeRows; ++r)
#pragma unroll
    for (int e = 0; e < CPT; ++e)
      if (r < nb && cvalid) us[r][ct + NT * e] = acc[r][e] * inv_l[r];
  __syncthreads();
  for (int r = 0; r < nb; ++r) {
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const f32x4 u0 = *(const f32x4*)(&us[r][64 * i + 8 * p]);
      const f32x4 u1 = *(const f32x4*)(&us[r][64 * i + 8 * p + 4]);
      dot = __builtin_fmaf(bf16_lo(wv[i][0]), u0[0], dot);
      dot = __builtin_fmaf(bf16_hi(wv[i][0]), u0[1], dot);
      dot = __builtin_fmaf(bf16_lo(wv[i][1]), u0[2], dot);
      dot = __builtin_fmaf(bf16_hi(wv[i][1]), u0[3], dot);
      dot = __builtin_fmaf(bf16_lo(wv[i][2]), u1[0], dot);
      dot = __builtin_fmaf(bf16_hi(wv[i][2]), u1[1], dot);
      dot = __builtin_fmaf(bf16_lo(wv[i][3]), u1[2], dot);
      dot = __builtin_fmaf(bf16_hi(wv[i][3]), u1[3], dot);
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    if (p == 0) {
      const int64_t idx = ((int64_t)(b0 + r) * a.H + h) * LHD + d;
      float v = dot;
      if (a.g) v *= sigmoidf_(bf16_to_f32(a.g[idx]));
      a.o[idx] = f32_to_bf16(v);
    }
  }
}

// Plain kernels around the templated body: the host pass then never instantiates the
// device-only builtins it uses.
__global__ __launch_bounds__(NT, 1) void latent_split_kernel_128(LatentDecodeArgs a) {
  latent_split_body<128>(a);
}
__global__ __launch_bounds__(NT, 1) void latent_split_kernel_256(LatentDecodeArgs a) {
  latent_split_body<256>(a);
}
__global__ __launch_bounds__(NT, 1) void latent_split_kernel_512(LatentDecodeArgs a) {
  latent_split_body<512>(a);
}

template <int DC>
hipError_t launch_latent_t(void (*split_kernel)(LatentDecodeArgs), const LatentDecodeArgs& a,
                           hipStream_t s) {
  hipLaunchKernelGGL((latent_absorb_kernel<DC>), dim3(DC / 64, a.H), dim3(NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nhb = (a.H + HB - 1) / HB;
  const long pg = ((long)a.splits * a.B + 7) / 8;  // groups of 8 range pairs
  const long npy = pg < 32768 ? pg : 32768;
  const long npz = (pg + npy - 1) / npy;
  hipLaunchKernelGGL(split_kernel, dim3(8 * nhb, (unsigned)npy, (unsigned)npz), dim3(NT), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = 4 * ((a.B + kMergeRows - 1) / kMergeRows);
  hipLaunchKernelGGL((latent_merge_kernel<DC>), dim3(8 * G, (a.H + 7) / 8), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_latent(const LatentDecodeArgs& a, hipStream_t s) {
  switch (a.DC) {
    case 128: return launch_latent_t<128>(latent_split_kernel_128, a, s);
    case 256: return launch_latent_t<256>(latent_split_kernel_256, a, s);
    case 512: return launch_latent_t<512>(latent_split_kernel_512, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmla
