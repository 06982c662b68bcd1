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
//    (K_{j+1} Q^T) and of this tile's values (V_j^T P_j^T) issue.  The iteration is a
//    fixed sequence of 32 MFMA groups, each holding one MFMA, the LDS reads of the
//    MFMA two groups on and a share of the softmax's vector work, kept in that order
//    by scheduling fences; the matrix cores, the vector ALU and LDS then work side by
//    side within a wave instead of in phases.
//  * K and V tiles go from global memory straight into LDS (buffer loads with the
//    LDS-direct form: no register staging, no vector ALU work).  Each load range ends
//    at the last valid row, so rows past the sequence end arrive as zeros with no
//    per-lane predicate.  Both tiles are row-major with the 16-byte chunks of each row
//    XOR-swizzled so that the fragment reads are free of bank conflicts.  A block's Q
//    rows take the same path once, at its start, and are read back as fragments.
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
//  * Per-sequence lengths (a packed batch of sequences of different lengths, offsets in
//    cu_q / cu_k on the device): a second instantiation of the same body reads each
//    sequence's rows and lengths at entry; its query i sits at position i + Tk_b - Tq_b.
//  * On a block's last tile a wave skips the 32-key halves that none of its queries may
//    see (their weights are exactly 0).
//  * Workgroups are mapped so that all query blocks of one head run on the same XCD
//    (shared L2); an XCD's heads go in groups of four (one group when the XCD has at
//    most three blocks per workgroup slot) whose query blocks launch heaviest (longest
//    prefix) first across the group.
#include <type_traits>
#include <utility>

#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int HD = 128;         // head width
constexpr int BM = 128;         // queries per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 256;   // 4 waves
constexpr int TILE = BN * HD;   // bf16 elements of one K or V tile (16 KB)
constexpr int KR = 3;           // fragment ring: LDS reads run two MFMA groups ahead
constexpr int kHeadGroup = 4;   // heads whose query blocks are interleaved in launch order
constexpr int kSlotsPerXcd = 64;  // workgroup slots of one XCD: 32 CUs x 2 workgroups
constexpr float kLazyRescale = 8.0f;   // raise the running max only past 2^8 growth
constexpr int kBufferDword3 = 0x00020000;  // raw buffer resource, 32-bit data format

// One array per buffer, so that the compiler can tell an LDS-direct load into one
// buffer from reads of another and does not wait for the load before those reads.
__shared__ __align__(16) bf16 lds_k0[TILE];
__shared__ __align__(16) bf16 lds_k1[TILE];
__shared__ __align__(16) bf16 lds_v0[TILE];
__shared__ __align__(16) bf16 lds_v1[TILE];
__shared__ __align__(16) bf16 lds_q[TILE];  // Q rows of waves 0 and 1 while a block starts
template <int B> __device__ __forceinline__ bf16* k_buf() { return B ? lds_k1 : lds_k0; }
template <int B> __device__ __forceinline__ bf16* v_buf() { return B ? lds_v1 : lds_v0; }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

template <int... Is, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, Is...>, F&& f) {
  (f(std::integral_constant<int, Is>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1, in order
template <int N, typename F> __device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}
// Hides a value from loop-invariant code motion (address arithmetic is redone per use).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

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

template <bool VARLEN, bool QLDS = true>
__device__ __forceinline__ void prefill_block(const PrefillArgs& a, const int b, const int h,
                                              const int qb);

template <bool VARLEN>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, int nqb, int total, int hgroup) {

  // ---- workgroup -> (head, query block).  Workgroups are dealt to the XCDs round-robin
  // and each XCD takes a contiguous set of heads (their K/V then share that XCD's L2).
  // Within an XCD, heads go in groups of `hgroup` and a group's query blocks in order
  // of decreasing work across its heads: launched in that order, the causal blocks
  // (2 to 2 nqb key tiles each) fill the XCD's workgroup slots evenly, where head by head
  // order left slots idle near each head's end.
  const int bid = blockIdx.x;
  const int per_xcd = total / kNumXcd;
  int head_lin, rank;
  if (!VARLEN && bid < per_xcd * kNumXcd && per_xcd % nqb == 0) {
    const int x = bid % kNumXcd, i = bid / kNumXcd;
    const int hx = per_xcd / nqb;  // heads per XCD
    const int G = min(hgroup, hx);
    const int g = i / (G * nqb), j = i % (G * nqb);
    const int gg = min(G, hx - g * G);  // heads in this group
    rank = j / gg;
    head_lin = x * hx + g * G + j % gg;
  } else {
    const int L = bid < per_xcd * kNumXcd ? (bid % kNumXcd) * per_xcd + bid / kNumXcd : bid;
    head_lin = L / nqb;
    rank = L % nqb;
  }
  const int qb = a.causal ? nqb - 1 - rank : rank;
  prefill_block<VARLEN>(a, head_lin / a.H, head_lin % a.H, qb);
}

// One query block: queries qb*BM .. qb*BM + BM - 1 of (batch b, head h), all key tiles it
// may see.  Leaves LDS in use until it returns (the caller separates two blocks with a
// barrier).  QLDS: the Q rows pass through LDS (a fifth 16 KB buffer, 80 KB per
// workgroup); the latent-fused kernel, whose workgroups need a little more LDS, loads
// them straight into registers.
template <bool VARLEN, bool QLDS>
__device__ __forceinline__ void prefill_block(const PrefillArgs& a, const int b, const int h,
                                              const int qb) {
  const int q0 = qb * BM;
  // Query rows, key rows and the position of query 0.  With per-sequence lengths
  // (packed rows, offsets in cu_q / cu_k) sequence b owns query rows cu_q[b] ..
  // cu_q[b+1] - 1 and key rows cu_k[b] .. cu_k[b+1] - 1; its query i sits at position
  // i + Tk_b - Tq_b.  The launch covers the longest sequence; blocks past a shorter
  // one's end leave at once.
  int T, Tk, off;
  int64_t qrow0;  // row of this sequence's query 0 in Q, G and O (as a token index)
  const bf16* __restrict__ Qh;
  const bf16* __restrict__ Kh;
  const bf16* __restrict__ Vh;
  if (VARLEN) {
    const int qlo = a.cu_q[b], klo = a.cu_k[b];
    T = a.cu_q[b + 1] - qlo;
    Tk = max(a.cu_k[b + 1] - klo, 0);
    if (q0 >= T) return;
    off = Tk - T;
    qrow0 = qlo;
    Qh = (const bf16*)a.q + (int64_t)qlo * a.qst + (int64_t)h * a.qsh;
    Kh = (const bf16*)a.k + (int64_t)klo * a.st + (int64_t)h * a.sh;
    Vh = (const bf16*)a.v + (int64_t)klo * a.st + (int64_t)h * a.sh;
  } else {
    T = a.T;
    Tk = a.Tk;
    off = a.Tk - a.T;
    qrow0 = (int64_t)b * a.T;
    const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
    Qh = (const bf16*)a.q + (int64_t)b * a.qsb + (int64_t)h * a.qsh;
    Kh = (const bf16*)a.k + head_off;
    Vh = (const bf16*)a.v + head_off;
  }

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS bases stay scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t st = a.st;

  // ---- this lane's query row and its Q fragments (B operand of S^T = K Q^T).  The
  // wave's 32 Q rows go to LDS as whole 256-byte rows (LDS-direct, like the tiles; waves
  // 0, 1 into lds_q, waves 2, 3 into V buffer 1, which the first iteration refills) and
  // come back as fragments after the first barrier.  16-byte register loads of one
  // query row per lane touch 32 rows per instruction and made a block's start ~2 us
  // longer (alternating runs, bitwise the same: B4 T1024 +4%, B1 T2048 gated +1%, B2
  // T4096 +0.3%).  Rows past the end arrive as zeros (the load range ends there).
  const int wq0 = q0 + wave * 32;  // first query of this wave
  const int tq = wq0 + l32;        // this lane's query
  bf16x8 qf[8];
  char* const q_lds = (char*)(wave < 2 ? lds_q : lds_v1) + (wave & 1) * 8192;
  const bool qlds = QLDS && 31 * a.qst + HD < ((int64_t)1 << 30);  // 32-bit offsets
  if (qlds) {
    const int qrows = min(32, T - wq0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Qh + (int64_t)wq0 * a.qst), (short)0,
        qrows > 0 ? (int)(((int64_t)(qrows - 1) * a.qst + HD) * 2) : 0, kBufferDword3);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 4 * u + (lane >> 4);
      load_lds16(r, (bf16*)(q_lds + u * 1024),
                 (uint32_t)((row * a.qst + k_chunk(row, lane & 15) * 8) * 2));
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (tq < T)
        qf[ks] = *(const bf16x8*)(Qh + (int64_t)tq * a.qst + ks * 16 + hh * 8);
      else
        qf[ks] = bf16x8{};
    }
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
  if (qlds) {
    // row l32, logical chunk 2 ks + hh (the K tiles' swizzle: conflict-free)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[ks] = *(const bf16x8*)(q_lds + l32 * 256 + (k_chunk(l32, 2 * ks + hh) << 4));
  }
  f32x16 s_cur[2];
  scores(B0{}, s_cur);
  if (0 >= mask_from) mask(s_cur, 0);
  float mt_cur = tile_max(s_cur);
  // tile 0 sets the running maximum (the output and sum are still zero, so the first
  // iteration needs no rescale)
  m_run = mt_cur;
  __syncthreads();  // every wave has read K buffer 0 before iteration 0 refills it

  // K fragment of (32-key half sub, k-step ks): row 32 sub + l32, logical chunk
  // 2 ks + hh, i.e. byte 8192 sub + (kfrag ^ 32 ks) of the tile (the swizzle only moves
  // bits 4..7).
  const int kfrag = l32 * 256 + ((hh ^ (l32 & 15)) << 4);

  // Output staging: each wave's 32 rows x 128 channels (bf16, 8 KB) in its own quarter of
  // the two K buffers, which no wave reads after the second-to-last tile.  With a gate,
  // the gate logits of those rows arrive there first: requested (whole 256-byte rows,
  // LDS-direct) when the last tile starts, so the epilogue finds them in LDS instead of
  // waiting for scattered 8-byte global reads.  Row r's 16-byte unit u sits at unit
  // u ^ (r mod 16) in both.
  char* const ep = (char*)(wave < 2 ? lds_k0 : lds_k1) + (wave & 1) * 8192;
  const int64_t hd = (int64_t)a.H * HD;
  const int grows = min(32, T - wq0);  // rows of this wave inside the sequence
  const bool gate_lds = a.g && grows > 0 && 31 * hd + HD < ((int64_t)1 << 30);
  auto load_gate = [&]() __attribute__((always_inline)) {
    const bf16* gbase = (const bf16*)a.g + (qrow0 + wq0) * hd + (int64_t)h * HD;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)gbase, (short)0, (int)(((int64_t)(grows - 1) * hd + HD) * 2), kBufferDword3);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = 4 * u + (lane >> 4);
      load_lds16(r, (bf16*)(ep + u * 1024),
                 (uint32_t)((row * hd + (((lane & 15) ^ (row & 15)) << 3)) * 2));
    }
  };

  // One iteration: weights of tile j, values of tile j, scores of tile j+1, as a fixed
  // interleave of 32 MFMA groups (the fences keep the order): each group issues one
  // MFMA, requests the LDS fragments of the MFMA two groups on, and carries a share of
  // the vector work (exponentials of tile j, then the maximum of tile j+1), so the
  // vector ALU and the LDS reads run under the matrix cores.
  //   NEXT: 0 = there is a next tile, 2 = tile j is the last one.
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
    // With per-sequence lengths a query may see no key at all (a sequence with more new
    // queries than keys): its maximum stays -inf and its weights must come out 0, not
    // 2^(-inf + inf).
    const float mneg = (VARLEN && m_run == -INFINITY) ? 0.0f : -m_run;
    if (NEXT != 2) {
      // next tiles in flight straight into LDS: K two tiles ahead (into the buffer K_j
      // used), V one tile ahead; tiles past the end arrive as zeros
      load_k(j + 2, BP{});
      load_v(j + 1, BQ{});
    }
    const char* kt = (const char*)k_buf<1 - PAR>();
    const bf16* vt = v_buf<PAR>();
    const int kfl = opaque(kfrag);
    auto kread = [&](auto I) __attribute__((always_inline)) -> bf16x8 {
      constexpr int i = decltype(I)::value;
      return *(const bf16x8*)(kt + (i >> 3) * 8192 + (kfl ^ ((i & 7) << 5)));
    };
    auto vread = [&](auto I) __attribute__((always_inline)) -> bf16x8 {
      constexpr int i = decltype(I)::value;
      const bf16* src = vt + (i >> 2) * 16 * HD + v_off[i & 3];
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)src);
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(src + 8 * HD));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // weights of two scores of tile j, rounded to bf16 (B operand of O^T = V^T P^T):
    // unit u covers elements 2 (u mod 4) + {0, 1} of half (u / 4) mod 2 of sub u / 8,
    // i.e. word u mod 4 of k-step u / 4
    uint32_t pw[4][4];
    auto eunit = [&](auto U) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      constexpr int sub = u >> 3, idx = ((u >> 2) & 1) * 8 + (u & 3) * 2;
      const float p0 = fast_exp2(__builtin_fmaf(s_cur[sub][idx], c2, mneg));
      const float p1 = fast_exp2(__builtin_fmaf(s_cur[sub][idx + 1], c2, mneg));
      bf16x2 pp;
      pp[0] = (bf16)p0;
      pp[1] = (bf16)p1;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones2, l_run, false);
      uint32_t w = __builtin_bit_cast(uint32_t, pp);
      // pin the unit where it is placed (the compiler would otherwise sink it past the
      // mask branch, next to its first use)
      asm volatile("" : "+v"(w), "+v"(l_run));
      pw[u >> 2][u & 3] = w;
    };
    auto pv_mfma = [&](auto I, const bf16x8& vf) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      u32x4 w;
      w[0] = pw[i >> 2][0];
      w[1] = pw[i >> 2][1];
      w[2] = pw[i >> 2][2];
      w[3] = pw[i >> 2][3];
      o_acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, w), o_acc[i & 3], 0, 0, 0);
    };

    if constexpr (NEXT == 2) {
      if (gate_lds) load_gate();
      // last tile: weights, then values.  A 32-key half past every key this wave's
      // queries may see holds only masked scores (weight exactly 0): its exponentials and
      // value MFMAs would add zeros, so the wave skips them.
      const int wlim = a.causal ? min(wq0 + 31 + off, Tk - 1) : Tk - 1;
      const bool live0 = j * BN <= wlim, live1 = j * BN + 32 <= wlim;
      if (live0) {
        static_for<8>([&](auto U) { eunit(U); });
        static_for<8>([&](auto I) { pv_mfma(I, vread(I)); });
      }
      if (live1) {
        static_for<8>([&](auto U) { eunit(std::integral_constant<int, decltype(U)::value + 8>{}); });
        static_for<8>([&](auto I) {
          constexpr int i = decltype(I)::value + 8;
          pv_mfma(std::integral_constant<int, i>{}, vread(std::integral_constant<int, i>{}));
        });
      }
    } else {
      f32x16 s_next[2];
      s_next[0] = f32x16{};
      s_next[1] = f32x16{};
      bf16x8 kf[KR], vf[KR];
      static_for<KR - 1>([&](auto I) { kf[decltype(I)::value] = kread(I); });
      __builtin_amdgcn_sched_barrier(0);
      // groups 0..15: scores of tile j+1 (K_{j+1} Q^T), weights units 0..9
      static_for<16>([&](auto G) {
        constexpr int g = decltype(G)::value;
        s_next[g >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g % KR], qf[g & 7], s_next[g >> 3], 0, 0, 0);
        constexpr int nx = g + KR - 1;  // fragment requested in this group
        if constexpr (nx < 16)
          kf[nx % KR] = kread(std::integral_constant<int, nx>{});
        else
          vf[(nx - 16) % KR] = vread(std::integral_constant<int, nx - 16>{});
        static_for<10>([&](auto U) {
          if constexpr ((decltype(U)::value * 16) / 10 == g) eunit(U);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      // the tiles that straddle the diagonal or the end (waits for the scores)
      if (j + 1 >= mask_from) mask(s_next, j + 1);
      __builtin_amdgcn_sched_barrier(0);
      // groups 16..21: values of tile j, weights units 10..15
      static_for<6>([&](auto G) {
        constexpr int g = decltype(G)::value;
        pv_mfma(G, vf[g % KR]);
        vf[(g + KR - 1) % KR] = vread(std::integral_constant<int, g + KR - 1>{});
        eunit(std::integral_constant<int, 10 + g>{});
        __builtin_amdgcn_sched_barrier(0);
      });
      // groups 22..31: values of tile j, maximum of tile j+1
      float mx0 = s_next[0][0], mx1 = s_next[1][0];
      static_for<10>([&](auto G) {
        constexpr int g = decltype(G)::value + 6;
        pv_mfma(std::integral_constant<int, g>{}, vf[g % KR]);
        if constexpr (g + KR - 1 < 16) vf[(g + KR - 1) % KR] = vread(std::integral_constant<int, g + KR - 1>{});
        if constexpr (g < 14) {
          constexpr int c = g - 6;  // 0..7: four-element chunk c mod 4 of sub c / 4
          if constexpr (c < 4) {
            mx0 = fmaxf(fmaxf(mx0, s_next[0][4 * c]), s_next[0][4 * c + 1]);
            mx0 = fmaxf(fmaxf(mx0, s_next[0][4 * c + 2]), s_next[0][4 * c + 3]);
          } else {
            mx1 = fmaxf(fmaxf(mx1, s_next[1][4 * (c - 4)]), s_next[1][4 * (c - 4) + 1]);
            mx1 = fmaxf(fmaxf(mx1, s_next[1][4 * (c - 4) + 2]), s_next[1][4 * (c - 4) + 3]);
          }
        }
        if constexpr (g == 14) mt_cur = swap_halves_max(fmaxf(mx0, mx1)) * c2;
        __builtin_amdgcn_sched_barrier(0);
      });
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

  // ---- epilogue: normalise, gate, round, store [B, T, H*128].  O^T leaves a lane four
  // consecutive channels of one query per register quad; stored directly, each store
  // instruction would touch 32 query rows.  Instead each wave puts its rows in the
  // staging area above and stores whole 256-byte rows from there (no bank conflicts on
  // either side).  A lane reads its gate logits from the very bytes it then overwrites.
  const float l_tot = swap_halves_sum(l_run);
  // (a query with no visible key, possible only with per-sequence lengths, writes zeros)
  const float inv = VARLEN ? (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) : 1.0f / l_tot;
  const bf16* __restrict__ gate =
      a.g && !gate_lds ? (const bf16*)a.g + (qrow0 + tq) * hd + (int64_t)h * HD : nullptr;
  if (gate_lds) __builtin_amdgcn_s_waitcnt(0);  // the gate rows have landed in LDS
#pragma unroll
  for (int dblk = 0; dblk < 4; ++dblk)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = dblk * 32 + 8 * r4 + 4 * hh;
      char* const slot = ep + l32 * 256 + (((d >> 3) ^ (l32 & 15)) << 4) + (d & 4) * 2;
      float v0 = o_acc[dblk][4 * r4 + 0] * inv;
      float v1 = o_acc[dblk][4 * r4 + 1] * inv;
      float v2 = o_acc[dblk][4 * r4 + 2] * inv;
      float v3 = o_acc[dblk][4 * r4 + 3] * inv;
      if (gate_lds || (gate && tq < T)) {
        const u32x2 gw = gate_lds ? *(const u32x2*)slot : *(const u32x2*)(gate + d);
        v0 *= sigmoidf_(bf16_lo(gw[0]));
        v1 *= sigmoidf_(bf16_hi(gw[0]));
        v2 *= sigmoidf_(bf16_lo(gw[1]));
        v3 *= sigmoidf_(bf16_hi(gw[1]));
      }
      u32x2 w;
      w[0] = pack_bf16x2(v0, v1);
      w[1] = pack_bf16x2(v2, v3);
      *(u32x2*)slot = w;
    }
  bf16* __restrict__ out = (bf16*)a.o + (qrow0 + wq0) * hd + (int64_t)h * HD;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int piece = lane + 64 * k;
    const int r = piece >> 4, u = piece & 15;  // query wq0 + r, channels 8u .. 8u+7
    const u32x4 v = *(const u32x4*)(ep + r * 256 + ((u ^ (r & 15)) << 4));
    if (wq0 + r < T) *(u32x4*)(out + r * hd + 8 * u) = v;
  }
}

// ---------------------------------------------------------------- latent-fused prefill
// Keys and values are rebuilt from the latent rows when attention runs ("Gated MLA",
// section "Start from familiar attention": K = C W_k^T, V = C W_v^T), each 128-row block
// once per head, inside the same launch as the attention: a persistent grid takes tasks
// from one counter per XCD, first the expansion tasks (batch, head, block) of that XCD's
// heads, then their query blocks (heaviest first).  A query block waits for the
// expansion blocks it reads; a task only waits for tasks taken before it from the same
// counter, and expansion tasks never wait, so every wait ends.  Expansion results go to
// a workspace and are read back through the XCD's L2.
constexpr int EXR = 128;      // latent rows (keys) per expansion task
constexpr int EXK = 32;       // latent channels per pipeline stage (64-byte LDS rows)
constexpr int kMaxSpins = 1 << 20;  // about a second: far beyond any expansion task

// Chunk swizzle of a 64-byte LDS row (four 16-byte chunks): rows 4i .. 4i+3 see chunk c at
// c ^ i mod 4, so 16 consecutive rows reading one chunk hit 16 distinct bank groups.
__device__ __forceinline__ int ex_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

// Keys and values of rows key0 .. key0 + 127 of batch b, head h:
// out[key][n] = sum_c C[key][c] W[n][c] for n < 128 from W_k,h (keys) and n >= 128 from
// W_v,h (values), on MFMA (D = W C^T: a lane holds four consecutive n of one key per
// register quad).  Wave w computes output columns 64 w .. 64 w + 63 for all 128 keys.
// Stages of 32 latent channels go global -> LDS (LDS-direct loads, two stages deep) in
// the attention's K buffers (C rows) and V buffers (W rows).
__device__ __forceinline__ void expand_block(const LatentPrefillArgs& f, int b, int h, int e) {
  const int T = f.p.T, H = f.p.H, DC = f.DC;
  const int key0 = e * EXR;
  const int rows = min(EXR, T - key0);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const bf16* Cb = f.c + ((int64_t)b * T + key0) * DC;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Cb, (short)0, rows * DC * 2, kBufferDword3);
  // waves 0, 1 load the 128 rows of W_k,h; waves 2, 3 those of W_v,h
  const bf16* Wb = (wave < 2 ? f.wk : f.wv) + (int64_t)h * HD * DC;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)Wb, (short)0, HD * DC * 2, kBufferDword3);
  // C stage: 128 rows x 64 B = 8 instructions of 16 rows, two per wave; W stage: 256 rows,
  // four per wave.  Lane i fills row (i / 4) of its 16-row group, physical chunk i mod 4.
  uint32_t coff[2], woff[4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = 16 * (2 * wave + u) + (lane >> 2);
    coff[u] = (uint32_t)(row * DC * 2 + ex_chunk(row, lane & 3) * 16);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = 16 * (4 * wave + u) + (lane >> 2);  // 0..255 over the four waves
    woff[u] = (uint32_t)((row & 127) * DC * 2 + ex_chunk(row, lane & 3) * 16);
  }
  auto load_stage = [&](int st, auto buf) __attribute__((always_inline)) {
    constexpr int P = decltype(buf)::value;
    const int koff = st * EXK * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rc, (lds_void_t*)(k_buf<P>() + (2 * wave + u) * 512), 16, coff[u], koff, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rw, (lds_void_t*)(v_buf<P>() + (4 * wave + u) * 512), 16, woff[u], koff, 0, 0);
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  // fragment of row r (of a stage's C or W rows), k-step ks: logical chunk 2 ks + hh
  auto frag = [&](const bf16* base, int r, int ks) __attribute__((always_inline)) -> bf16x8 {
    return *(const bf16x8*)((const char*)base + r * 64 + ex_chunk(r, 2 * ks + hh) * 16);
  };
  auto compute = [&](auto buf) __attribute__((always_inline)) {
    constexpr int P = decltype(buf)::value;
    const bf16* cs = k_buf<P>();
    const bf16* ws = v_buf<P>();
#pragma unroll
    for (int ks = 0; ks < EXK / 16; ++ks) {
      bf16x8 wf[2], cf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) wf[i] = frag(ws, 64 * wave + 32 * i + l32, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) cf[j] = frag(cs, 32 * j + l32, ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], cf[j], acc[i][j], 0, 0, 0);
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int ns = DC / EXK;
  load_stage(0, B0{});
  for (int st = 0; st < ns; st += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // stage st landed; every wave is done with stage st - 1
    if (st + 1 < ns) load_stage(st + 1, B1{});
    compute(B0{});
    if (st + 1 < ns) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (st + 2 < ns) load_stage(st + 2, B0{});
      compute(B1{});
    }
  }
  // rows key0 + 32 j + l32; columns n = 64 w + 32 i + 8 (r / 4) + 4 hh + r mod 4
  bf16* out = (wave < 2 ? f.kws : f.vws) + (int64_t)h * HD;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int key = 32 * j + l32;
    if (key >= rows) continue;
    bf16* orow = out + ((int64_t)b * T + key0 + key) * ((int64_t)H * HD);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int n = (64 * wave + 32 * i + 8 * r4 + 4 * hh) & 127;
        u32x2 v;
        v[0] = pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]);
        v[1] = pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
        *(u32x2*)(orow + n) = v;
      }
  }
}

// The accelerator die (XCD) this workgroup runs on, from the hardware register XCC_ID.
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (kNumXcd - 1);
}

// Heads are dealt to the XCDs (head_lin mod 8); each XCD takes the tasks of its heads from
// its own counter: first their expansion blocks, then their query blocks, heaviest first.
// A head's keys and values are therefore written and read through one die's L2, which is
// coherent for all of its compute units: the producer only waits for its stores to reach
// L2 before raising the flag, and the consumer reads the flag around the caches
// (agent-scope atomics), with no cache writeback or invalidation on either side.
__global__ __launch_bounds__(NTHREADS, 2) void prefill_latent_kernel(LatentPrefillArgs f) {
  __shared__ int task_slot;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int heads = f.p.B * f.p.H;
  const int x = xcd_id();
  const int nh = (heads - x + kNumXcd - 1) / kNumXcd;  // heads head_lin = x + 8 i
  const int n_e = nh * f.nE;
  const int n_all = n_e + nh * f.nqb;
  int* const counter = f.counter + x;
  for (;;) {
    __syncthreads();  // the previous task is done with LDS and task_slot
    if (tid == 0)
      task_slot = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = task_slot;
    if (t >= n_all) break;
    if (t < n_e) {
      // expansion task: head-major, so a head's blocks are done together
      const int head_lin = x + kNumXcd * (t / f.nE), e = t % f.nE;
      expand_block(f, head_lin / f.p.H, head_lin % f.p.H, e);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are in L2
      __syncthreads();                // ... and every other wave's
      if (tid == 0)
        __hip_atomic_store(f.flags + (int64_t)head_lin * f.nE + e, 1, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // query block, heaviest first across this XCD's heads
      const int u = t - n_e;
      const int rank = u / nh;
      const int head_lin = x + kNumXcd * (u % nh);
      const int qb = f.p.causal ? f.nqb - 1 - rank : rank;
      const int T = f.p.T;
      const int last = f.p.causal ? min(T - 1, qb * BM + BM - 1) : T - 1;
      const int need = last / EXR + 1;  // expansion blocks 0 .. need - 1
      if (tid < 64) {
        const int* fl = f.flags + (int64_t)head_lin * f.nE;
        for (int e = lane; e < need; e += 64) {
          int spins = 0;
          while (__hip_atomic_load(fl + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins > kMaxSpins) {  // cannot happen: the task is older than this one
              __hip_atomic_store(f.error, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
          }
        }
      }
      __syncthreads();
      prefill_block<false, false>(f.p, head_lin / f.p.H, head_lin % f.p.H, qb);
    }
  }
}

// Clears the ready flags and the task counter (a kernel, not a memset, so the call stays
// capturable in a graph).
__global__ __launch_bounds__(256) void prefill_latent_clear_kernel(int* flags, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) flags[i] = 0;
}

// Plain kernels around the templated body (the host pass then never instantiates the
// device-only builtins it uses).
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a, int nqb,
                                                                   int total, int hgroup) {
  prefill_body<false>(a, nqb, total, hgroup);
}
__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_varlen_kernel(PrefillArgs a, int nqb,
                                                                          int total, int hgroup) {
  prefill_body<true>(a, nqb, total, hgroup);
}

}  // namespace

hipError_t launch_prefill_bf16_varlen(const PrefillArgs& a, hipStream_t s) {
  // a.T is the longest query sequence: every sequence gets that many query blocks and the
  // blocks past its own end leave at once; each (sequence, head) stays on one XCD
  const int nqb = (a.T + BM - 1) / BM;
  const long total = (long)nqb * a.B * a.H;
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_bf16_varlen_kernel, dim3((unsigned)total), dim3(NTHREADS), 0, s, a,
                     nqb, (int)total, 1);
  return hipGetLastError();
}

hipError_t launch_prefill_latent(const LatentPrefillArgs& f, int workgroups, hipStream_t s) {
  // flags, the eight per-XCD counters and the error word are contiguous in the workspace
  const int n = f.ntasks_e + kNumXcd + 1;
  hipLaunchKernelGGL(prefill_latent_clear_kernel, dim3((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024),
                     dim3(256), 0, s, f.flags, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(prefill_latent_kernel, dim3(workgroups), dim3(NTHREADS), 0, s, f);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16_mfma(const PrefillArgs& a, hipStream_t s) {
  const int nqb = (a.T + BM - 1) / BM;
  const long total = (long)nqb * a.B * a.H;
  if (total > 0x7fffffffL) return hipErrorInvalidConfiguration;
  // Heads are grouped by four (their K/V stay in the XCD's L2 while the group runs); when
  // an XCD has at most three workgroups per slot in all, its heads form one group, so the
  // whole launch runs heaviest first and the last blocks end together (measured: +5% at
  // B1 T2048, +2% at B1 T1024; at six rounds or more, one group loses 2-12%).
  const long per_xcd = total / kNumXcd;
  const int hgroup = per_xcd <= 3 * kSlotsPerXcd ? (int)per_xcd : kHeadGroup;
  hipLaunchKernelGGL(prefill_bf16_kernel, dim3((unsigned)total), dim3(NTHREADS), 0, s, a, nqb,
                     (int)total, hgroup);
  return hipGetLastError();
}

}  // namespace gmla
