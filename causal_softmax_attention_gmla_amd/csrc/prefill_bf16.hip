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
//  * K tiles sit in LDS row-major; V tiles are written to LDS transposed (V^T), with
//    the keys of every 16-key group permuted so that each A-operand fragment is one
//    16-byte LDS read.  Row paddings make both the fragment reads and the transposing
//    writes free of bank conflicts.  Two buffers each; one barrier per tile.
//  * Global loads are buffer loads whose range ends at the last valid row: rows
//    past the sequence end read as zero without any per-lane predicate.
//  * Online softmax in base 2 (scale * log2 e folded into one FMA); a row's running
//    maximum is only raised when the tile's maximum exceeds it by more than 2^8,
//    which skips most O rescales; the stale maximum scales numerator and
//    denominator alike, so the result is unchanged.
//  * Causal tiles above the diagonal are never loaded; the mask is an index compare
//    applied only on the two tiles that straddle the diagonal or the sequence end.
//  * Workgroups are mapped so that all query blocks of one head run on the same XCD
//    (shared L2), heaviest (longest-prefix) blocks first.
#include "gmla_internal.h"

namespace gmla {
namespace {

constexpr int HD = 128;         // head width
constexpr int BM = 128;         // queries per workgroup
constexpr int BN = 64;          // keys per tile
constexpr int NTHREADS = 256;   // 4 waves
constexpr int K_LD = HD + 8;    // K tile row stride (bf16): 272 B rows
constexpr int VT_LD = BN + 8;   // V^T tile row stride (bf16): 144 B rows
constexpr int K_TILE = BN * K_LD;
constexpr int VT_TILE = HD * VT_LD;
constexpr float kLazyRescale = 8.0f;   // raise the running max only past 2^8 growth
constexpr int kBufferDword3 = 0x00020000;  // raw buffer resource, 32-bit data format

struct __align__(16) Smem {
  bf16 k[2][K_TILE];
  bf16 vt[2][VT_TILE];
};

// Key slot inside a 16-key group of the V^T tile: keys 4..7 and 8..11 trade places,
// so that slots 8h .. 8h+7 hold exactly the keys that lane half h feeds to the
// O^T MFMA from its S^T accumulator registers (keys 4h..4h+3 and 8+4h..8+4h+3).
__device__ __forceinline__ int key_group_slot(int g4) { return g4 == 1 ? 2 : (g4 == 2 ? 1 : g4); }

__device__ __forceinline__ float swap_halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over rows [tile*BN, tile*BN + BN) of one head; rows at or past T
// (and whole tiles past the end) fall outside its range and load as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* head, int tile, int T,
                                                           int64_t st) {
  const int rows = min(BN, T - tile * BN);
  const int bytes = rows > 0 ? (int)(((int64_t)(rows - 1) * st + HD) * 2) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)(head + (int64_t)tile * BN * st), (short)0, bytes,
                                           kBufferDword3);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__global__ __launch_bounds__(NTHREADS, 2) void prefill_bf16_kernel(PrefillArgs a, int nqb,
                                                                   int total) {
  __shared__ Smem sm;

  // ---- workgroup -> (head, query block): same-head blocks on one XCD, heavy first
  const int bid = blockIdx.x;
  const int per_xcd = total / kNumXcd;
  const int L = bid < per_xcd * kNumXcd ? (bid % kNumXcd) * per_xcd + bid / kNumXcd : bid;
  const int head_lin = L / nqb;
  const int qb = a.causal ? nqb - 1 - (L % nqb) : (L % nqb);
  const int b = head_lin / a.H;
  const int h = head_lin % a.H;
  const int q0 = qb * BM;
  const int T = a.T;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int64_t head_off = (int64_t)b * a.sb + (int64_t)h * a.sh;
  const bf16* __restrict__ Qh = (const bf16*)a.q + head_off;
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
      qf[ks] = *(const bf16x8*)(Qh + (int64_t)tq * st + ks * 16 + hh * 8);
    else
      qf[ks] = bf16x8{};
  }

  // ---- key tiles this workgroup visits
  const int nkt_all = (T + BN - 1) / BN;
  const int ntiles = a.causal ? min(nkt_all, (q0 + BM) / BN) : nkt_all;
  // first tile that needs the index mask: the diagonal pair (causal) or the tail
  const int mask_from = a.causal ? ntiles - 2 : (T % BN ? ntiles - 1 : ntiles);

  // per-thread byte offsets of the staged rows inside a tile (constant per tile)
  uint32_t koff[4], voff[4];
  const int v_kg = tid & 15;   // value key group: keys 4*v_kg .. 4*v_kg+3
  const int v_c16 = tid >> 4;  // value channel chunk: channels 8*v_c16 .. +7
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * NTHREADS + tid;
    koff[i] = (uint32_t)(((id >> 4) * st + (id & 15) * 8) * 2);
    voff[i] = (uint32_t)(((v_kg * 4 + i) * st + v_c16 * 8) * 2);
  }
  const int vt_slot = (v_kg >> 2) * 16 + key_group_slot(v_kg & 3) * 4;

  u32x4 kreg[4], vreg[4];
  auto load_k = [&](int tile) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Kh, tile, T, st);
#pragma unroll
    for (int i = 0; i < 4; ++i) kreg[i] = buffer_load16(r, koff[i]);
  };
  auto load_v = [&](int tile) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(Vh, tile, T, st);
#pragma unroll
    for (int i = 0; i < 4; ++i) vreg[i] = buffer_load16(r, voff[i]);
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = i * NTHREADS + tid;
      *(u32x4*)(&sm.k[buf][(id >> 4) * K_LD + (id & 15) * 8]) = kreg[i];
    }
  };
  // transpose 4 keys x 8 channels into 8 channels x 4 keys (8-byte LDS writes); the
  // 16 lanes that share a channel chunk write one full 128-byte V^T row
  auto store_v = [&](int buf) {
    bf16* base = &sm.vt[buf][(v_c16 * 8) * VT_LD + vt_slot];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x0 = vreg[0][w], x1 = vreg[1][w], x2 = vreg[2][w], x3 = vreg[3][w];
      u32x2 even, odd;
      even[0] = (x0 & 0xffffu) | (x1 << 16);
      even[1] = (x2 & 0xffffu) | (x3 << 16);
      odd[0] = (x0 >> 16) | (x1 & 0xffff0000u);
      odd[1] = (x2 >> 16) | (x3 & 0xffff0000u);
      *(u32x2*)(base + (2 * w) * VT_LD) = even;
      *(u32x2*)(base + (2 * w + 1) * VT_LD) = odd;
    }
  };
  // S^T = K Q^T for the 64 keys of a K buffer (two 32-key halves)
  auto scores = [&](int buf, f32x16* s) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      s[sub] = f32x16{};
      const bf16* krow = &sm.k[buf][(sub * 32 + l32) * K_LD + hh * 8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *(const bf16x8*)(krow + ks * 16);
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[sub], 0, 0, 0);
      }
    }
  };

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
  const int lim = a.causal ? min(tq, T - 1) : T - 1;  // last key this query may see

  // ---- prologue: K0, V0 and K1 in LDS; scores of tile 0
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  load_k(1);
  store_k(1);
  __syncthreads();
  f32x16 s_cur[2];
  scores(0, s_cur);
  __syncthreads();  // every wave has read K buffer 0 before iteration 0 refills it

  for (int j = 0; j < ntiles; ++j) {
    // next loads in flight: K two tiles ahead, V one tile ahead (zero past the end)
    load_k(j + 2);
    load_v(j + 1);

    const int kbase = j * BN;
    if (j >= mask_from) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + sub * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) s_cur[sub][r] = -INFINITY;
        }
    }
    // tile maximum of this query (both halves)
    float mx = fmaxf(s_cur[0][0], s_cur[0][1]);
#pragma unroll
    for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s_cur[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_cur[1][r]);
    mx = swap_halves_max(mx);
    const float mt = mx * c2;
    const bool grow = mt > m_run + kLazyRescale;
    if (__any(grow)) {
      // only the lanes whose maximum grew move it; the others keep theirs
      // exactly (alpha = 1), so a row never depends on its neighbours' scores
      const float alpha = grow ? fast_exp2(m_run - mt) : 1.0f;  // m_run = -inf: 0
      m_run = grow ? mt : m_run;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[i][r] *= alpha;
    }
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
    // scores of the next tile (its K is already in LDS)
    f32x16 s_next[2];
    scores((j + 1) & 1, s_next);
    // O^T += V^T P^T over the tile's 64 keys (4 k-steps of 16), 4 blocks of 32 channels
    const int vb = j & 1;
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const bf16x8 pb = p[kstep >> 1][kstep & 1];
#pragma unroll
      for (int dblk = 0; dblk < 4; ++dblk) {
        const bf16x8 vf =
            *(const bf16x8*)(&sm.vt[vb][(dblk * 32 + l32) * VT_LD + (kstep * 2 + hh) * 8]);
        o_acc[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o_acc[dblk], 0, 0, 0);
      }
    }
    // stage K_{j+2} (into the buffer K_j used) and V_{j+1}
    store_k(j & 1);
    store_v((j + 1) & 1);
    __syncthreads();
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
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
