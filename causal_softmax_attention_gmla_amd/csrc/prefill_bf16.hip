// Causal softmax attention, bf16 inputs, head width 128, MFMA (gfx950).
//
// Computes per head ("Gated MLA", section "Start from familiar attention";
// "Kimi K3 - Softmax over keys", the softmax formula; "Kimi K2 - Construct causal
// mask", the formula for M):
//     O[t,:] = sum_{s <= t} softmax_s(scale * q_t . k_s) v_s
// with the softmax in float32, then optionally multiplies each output channel by
// sigmoid(G) ("Gated MLA", section "The channel-wise output gate").
//
// Design (one workgroup = 128 queries of one (batch, head), 4 waves of 32 queries):
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16.
//    In the 32x32 accumulator, lane l then holds 16 keys of query (l mod 32), so the
//    row maximum and row sum of a query are lane-local except for one exchange
//    between the two 32-lane halves (v_permlane32_swap).
//  * The value product is computed transposed too, O^T = V^T P^T.  Its B operand is
//    P^T, and the S^T accumulator registers are already laid out as that operand
//    (after f32 -> bf16 rounding): no shuffles.  O^T keeps each query's 128 output
//    channels in that query's lanes, so rescaling by the running maximum is
//    lane-local as well.
//  * Software pipeline: keys run one tile ahead of values.  Iteration j turns the
//    scores of tile j into weights while the MFMAs of the next tile's scores
//    (K_{j+1} Q^T) and of this tile's values (V_j^T P_j^T) issue, so the vector
//    ALU work of the softmax overlaps the matrix cores.
//  * K and V tiles go from global memory straight into LDS (buffer loads with the
//    LDS-direct form: no register staging, no vector ALU work).  Each load range ends
//    at the last valid row, so rows past the sequence end arrive as zeros with no
//    per-lane predicate.  Both tiles are row-major with the 16-byte chunks of each row
//    XOR-swizzled so that the fragment reads are free of bank conflicts.
//  * The value operand is read with the transposing LDS load ds_read_b64_tr_b16:
//    each 16-lane group gathers 16 consecutive channels of 4 keys, which is exactly
//    the A-operand layout of O^T = V^T P^T for the keys the lane's P^T registers hold.
//    Two buffers per tile kind; one barrier per tile.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA); a row's running
//    maximum is only raised when the tile's maximum exceeds it by more than 2^8,
//    which skips most O rescales; the stale maximum scales numerator and
//    denominator alike, so the result is unchanged.
//  * Causal tiles above the diagonal are never loaded; the mask is an index compare
//    applied only on the tiles that straddle the diagonal or the sequence end.
//  * The queries may be the last T rows of Tk >= T keys (a chunk after a cache):
//    query i sits at position i + Tk - T and sees the keys up to there ("Kimi K2 -
//    Construct causal mask": positions continue from the cached length).
//  * Workgroups are mapped so that all query blocks of one head run on the same XCD
//    (shared L2), heaviest (longest-prefix) blocks first.
#include <type_traits>

#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int HD = 128;         // head width
constexpr int BM = 128;         // queries per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 256;   // 4 waves
constexpr int TILE = BN * HD;   // bf16 elements of one K or V tile (16 KB)
constexpr float kLazyRescale = 8.0f;   // raise the running max only past 2^8 growth
constexpr int kBufferDword3 = 0x00020000;  // raw buffer resource, 32-bit data format

// One array per buffer, so that the compiler can tell an LDS-direct load into one
// buffer from reads of another and does not wait for the load before those reads.
__shared__ __align__(16) bf16 lds_k0[TILE];
__shared__ __align__(16) bf16 lds_k1[TILE];
__shared__ __align__(16) bf16 lds_v0[TILE];
__shared__ __align__(16) bf16 lds_v1[TILE];
template <int B> __device__ __forceinline__ bf16* k_buf() { return B ? lds_k1 : lds_k0; }
template <int B> __device__ __forceinline__ bf16* v_buf() { return B ? lds_v1 : lds_v0; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// Swizzles of the 16-byte chunk index (8 channels) inside a 256-byte tile row.
// K: 16 consecutive rows read the same logical chunk -> 16 distinct bank groups.
// V: the transposing reads of one lane half touch 4 consecutive rows x 4 chunks.
__device__ __forceinline__ int k_chunk(int row, int c) { return c ^ (row & 15); }
__device__ __forceinline__ int v_chunk(int row, int c) { return c ^ ((row & 3) << 2); }

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over rows [tile*BN, tile*BN + BN) of one head; key rows at or past
// Tk (and whole tiles past the end) fall outside its range and load as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* head, int tile, int Tk,
                                                           int64_t st) {
  const int rows = min(BN, Tk - tile * BN);
  const int bytes = rows > 0 ? (int)(((int64_t)(rows - 1) * st + HD) * 2) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (int64_t)tile * BN * st), (short)0, bytes,
                                           kBufferDword3);
}

// 64 lanes x 16 bytes from global (lane's own byte offset) into 1 KB of LDS at dst,
// lane i's bytes landing at dst + 16 i.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, bf16* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 16, off, 0, 0, 0);
}

__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a, int nqb,
                                                                   int total) {

  // ---- workgroup -> (head, query block): same-head blocks on one XCD, heavy first
  const int bid = blockIdx.x;
  const int per_xcd = total / kNumXcd;
  const int L = bid < per_xcd * kNumXcd ? (bid % kNumXcd) * per_xcd + bid / kNumXcd : bid;
  const int head_lin = L / nqb;
  const int qb = a.causal ? nqb - 1 - (L % nqb) : (L % nqb);
  const int b = head_lin / a.H;
  const int h = head_lin % a.H;
  const int q0 = qb * BM;
  const int T = a.T;             // query rows
  const int Tk = a.Tk;           // key rows
  const int off = a.Tk - a.T;    // position of query 0

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16* __restrict__ Qh = (const bf16*)a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh;
  const bf16* __restrict__ Kh = (const bf16*)a.k + head_off;
  const bf16* __restrict__ Vh = (const bf16*)a.v + head_off;
  const int64_t st = a.st;

  // ---- this lane's query row and its Q fragments (B operand of S^T = K Q^T)
  const int wq0 = q0 + wave * 32;  // first query of this wave
  const int tq = wq0 + l32;        // this lane's query
  bf16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (tq < T)
      qf[ks] = *(const bf16x8*)(Qh + (int64_t)tq * a.qst + ks * 16 + hh * 8);
    else
      qf[ks] = bf16x8{};
  }

  // ---- key tiles this workgroup visits
  const int nkt_all = (Tk + BN - 1) / BN;
  const int ntiles = a.causal ? min(nkt_all, (q0 + BM - 1 + off) / BN + 1) : nkt_all;
  // first tile that needs the index mask: the one holding the key just after the
  // block's first query (causal; the diagonal band and the tail follow it), or the
  // ragged tail (non-causal)
  const int mask_from =
      a.causal ? min(ntiles, (q0 + off + 1) / BN) : (Tk % BN ? ntiles - 1 : ntiles);

  // Tile staging: each wave moves 4 KB of a tile (4 loads of 64 lanes x 16 bytes).
  // Load u of wave w fills LDS rows 4m .. 4m+3 (m = 4w + u) in physical chunk order;
  // lane i therefore fetches row 4m + i/16, logical chunk (i mod 16) ^ swizzle(row).
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 4 * (wave * 4 + u) + (lane >> 4);
    koff[u] = (uint32_t)((row * st + k_chunk(row, lane & 15) * 8) * 2);
    voff[u] = (uint32_t)((row * st + v_chunk(row, lane & 15) * 8) * 2);
  }
  auto load_k = [&](int tile, auto buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Kh, tile, Tk, st);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      load_lds16(r, k_buf<decltype(buf)::value>() + (wave * 4 + u) * 512, koff[u]);
  };
  auto load_v = [&](int tile, auto buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Vh, tile, Tk, st);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      load_lds16(r, v_buf<decltype(buf)::value>() + (wave * 4 + u) * 512, voff[u]);
  };
  // wait for this wave's LDS-direct loads, then for every wave
  auto tile_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // S^T = K Q^T for the 64 keys of a K buffer (two 32-key halves)
  auto scores = [&](auto buf, f32x16* s) __attribute__((always_inline)) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub] = f32x16{};
      const int row = sub * 32 + l32;
      const bf16* krow = k_buf<decltype(buf)::value>() + row * HD;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(krow + k_chunk(row, ks * 2 + hh) * 8);
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[sub], 0, 0, 0);
      }
    }
  };

  // Transposed value reads: in each 16-lane group (lane p = lane mod 16) lane p points
  // at key 4*hh + p/4 (and that + 8), channels dbase + 4*(p mod 4) .. +3, with dbase =
  // 32*dblk + 16*((lane/16) mod 2); the hardware then hands lane p channel dbase + p
  // of those 4 keys: keys 16*kstep + 4*hh + {0..3, 8..11} for channel 32*dblk + (lane
  // mod 32), matching the keys of this lane's P^T registers.
  int v_off[4];
  {
    const int p = lane & 15;
    const int row = 4 * hh + (p >> 2);
#pragma unroll
    for (int dblk = 0; dblk < 4; ++dblk) {
      const int d0 = dblk * 32 + 16 * ((lane >> 4) & 1) + 4 * (p & 3);
      v_off[dblk] = row * HD + v_chunk(row, d0 >> 3) * 8 + (d0 & 7);
    }
  }

  // ---- accumulators
  f32x16 o_acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o_acc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of scores, base-2 units
  float l_run = 0.0f;       // running sum of bf16-rounded weights (this half's keys)
  const float c2 = a.scale * kLog2e;
  bf16x2 ones2;
  ones2[0] = (bf16)1.0f;
  ones2[1] = (bf16)1.0f;
  const int lim = a.causal ? min(tq + off, Tk - 1) : Tk - 1;  // last key this query may see

  // keys after the query (causal) or past the sequence end score -inf
  auto mask = [&](f32x16* s, int tile) __attribute__((always_inline)) {
    const int kbase = tile * BN;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + sub * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (key > lim) s[sub][r] = -INFINITY;
      }
  };
  // this query's maximum over a tile (both lane halves), in base-2 units
  auto tile_max = [&](const f32x16* s) __attribute__((always_inline)) {
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    return swap_halves_max(mx) * c2;
  };

  // ---- prologue: K0, V0 and K1 in LDS; scores and maximum of tile 0
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  load_k(0, B0{});
  load_v(0, B0{});
  load_k(1, B1{});
  tile_barrier();
  f32x16 s_cur[2];
  scores(B0{}, s_cur);
  if (0 >= mask_from) mask(s_cur, 0);
  float mt_cur = tile_max(s_cur);
  __syncthreads();  // every wave has read K buffer 0 before iteration 0 refills it

  // One iteration: weights of tile j, values of tile j, scores of tile j+1.
  //   NEXT: 0 = there is a next tile (masked if it straddles the diagonal or the end),
  //         2 = tile j is the last one.
  //   PAR = j mod 2 selects the buffers: K_{j+1} and V_j are read, K_{j+2} and V_{j+1}
  //   are loaded into the buffers K_j and V_{j-1} used.
  auto step = [&](int j, auto next_kind, auto parity) __attribute__((always_inline)) {
    constexpr int NEXT = decltype(next_kind)::value;
    constexpr int PAR = decltype(parity)::value;
    using BP = std::integral_constant<int, PAR>;
    using BQ = std::integral_constant<int, 1 - PAR>;
    const bool grow = mt_cur > m_run + kLazyRescale;
    if (__any(grow)) {
      // only the lanes whose maximum grew move it; the others keep theirs
      // exactly (alpha = 1), so a row never depends on its neighbours' scores
      const float alpha = grow ? fast_exp2(m_run - mt_cur) : 1.0f;  // m_run = -inf: 0
      m_run = grow ? mt_cur : m_run;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[i][r] *= alpha;
    }
    if (NEXT != 2) {
      // next tiles in flight straight into LDS: K two tiles ahead (into the buffer K_j
      // used), V one tile ahead; tiles past the end arrive as zeros
      load_k(j + 2, BP{});
      load_v(j + 1, BQ{});
    }
    // scores of the next tile (its K is already in LDS)
    f32x16 s_next[2];
    if (NEXT != 2) scores(BQ{}, s_next);
    // weights, rounded to bf16 as the B operand of O^T = V^T P^T
    bf16x8 p[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = fast_exp2(__builtin_fmaf(s_cur[sub][half * 8 + e], c2, -m_run));
          const float p1 = fast_exp2(__builtin_fmaf(s_cur[sub][half * 8 + e + 1], c2, -m_run));
          bf16x2 pp;
          pp[0] = (bf16)p0;
          pp[1] = (bf16)p1;
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, l_run, false);
          p[sub][half][e] = pp[0];
          p[sub][half][e + 1] = pp[1];
        }
    // O^T += V^T P^T over the tile's 64 keys (4 k-steps of 16), 4 blocks of 32 channels
    const bf16* vtile = v_buf<PAR>();
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const bf16x8 pb = p[kstep >> 1][kstep & 1];
#pragma unroll
      for (int dblk = 0; dblk < 4; ++dblk) {
        const bf16* src = vtile + kstep * 16 * HD + v_off[dblk];
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(src + 8 * HD));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o_acc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o_acc[dblk], 0, 0, 0);
      }
    }
    if (NEXT != 2) {
      if (j + 1 >= mask_from) mask(s_next, j + 1);
      mt_cur = tile_max(s_next);
      tile_barrier();
      s_cur[0] = s_next[0];
      s_cur[1] = s_next[1];
    }
  };

  using NotLast = std::integral_constant<int, 0>;
  using Last = std::integral_constant<int, 2>;
  int j = 0;
  for (; j + 2 < ntiles; j += 2) {  // j even: buffers alternate with the parity of j
    step(j, NotLast{}, B0{});
    step(j + 1, NotLast{}, B1{});
  }
  if (j + 1 < ntiles) {
    step(j, NotLast{}, B0{});
    step(j + 1, Last{}, B1{});
  } else {
    step(j, Last{}, B0{});
  }

  // ---- epilogue: normalise, gate, round, store [B, T, H*128]
  if (tq >= T) return;
  const float l_tot = swap_halves_sum(l_run);
  const float inv = 1.0f / l_tot;
  const int64_t row = ((int64_t)b * T + tq) * ((int64_t)a.H * HD) + (int64_t)h * HD;
  bf16* __restrict__ out = (bf16*)a.o + row;
  const bf16* __restrict__ gate = a.g ? (const bf16*)a.g + row : nullptr;
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = dblk * 32 + 8 * r4 + 4 * hh;
      float v0 = o_acc[dblk][4 * r4 + 0] * inv;
      float v1 = o_acc[dblk][4 * r4 + 1] * inv;
      float v2 = o_acc[dblk][4 * r4 + 2] * inv;
      float v3 = o_acc[dblk][4 * r4 + 3] * inv;
      if (gate) {
        const u32x2 gw = *(const u32x2*)(gate + d);
        v0 *= sigmoidf_(bf16_lo(gw[0]));
        v1 *= sigmoidf_(bf16_hi(gw[0]));
        v2 *= sigmoidf_(bf16_lo(gw[1]));
        v3 *= sigmoidf_(bf16_hi(gw[1]));
      }
      u32x2 w;
      w[0] = pack_bf16x2(v0, v1);
      w[1] = pack_bf16x2(v2, v3);
      *(u32x2*)(out + d) = w;
    }
}

}  // namespace

hipError_t launch_prefill_bf16_mfma(const PrefillArgs& a, hipStream_t s) {
  const int nqb = (a.T + BM - 1) / BM;
  const long total = (long)nqb * a.B * a.H;
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)total), dim3(NTHREADS), 0, s, a, nqb,
                     (int)total);
  return hipGetLastError();
}

}  // namespace gmla
