// Exact attention backward (dQ, dK, dV) for MI355X / gfx950 (CDNA4).
//
// The gradients of O = softmax(s Q K^T) V for dL/dO = dO, per (batch, head) slice:
//   P = exp(s Q K^T - LSE)   (rows; recomputed from the LSE the forward returned)
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
//   dQ = s dS K,  dK = s dS^T Q.
// "CUDA 算子工程：手写 FlashAttention v2 之路" ch. 14 §14.5 notes that the forward keeps
// the LSE for this pass, and §14.7 that FA2's backward runs K/V-stationary (outer loop
// over K/V blocks, inner over Q blocks) with dQ accumulated by atomics. Here dQ has a
// kernel of its own instead, Q-stationary like the forward: both kernels recompute
// P from the LSE, so no atomics, no fp32 dQ buffer, and the result is deterministic.
//
// Two launches on the caller's stream:
//   1. fa_bwd_dq_kernel: a workgroup pins 128 query rows (4 waves x 32) with Q^T and
//      dO^T in registers, forms D_i = dO_i . O_i and the LSE in base-2 units
//      (LSE_i log2 e, +inf for a row that sees no key) of its rows and leaves -D and
//      that LSE, fp32, in the caller's workspace; then it streams K and V in tiles of
//      32 keys through LDS:
//        S^T = K Q^T, dP^T = V dO^T            (MFMA, K and V rows from LDS)
//        P^T = 2^(c S^T - LSE log2 e), dS^T = P^T * (dP^T - D)   (VALU)
//        dQ^T += K^T dS^T                      (MFMA, K^T by transposing LDS reads)
//   2. fa_bwd_dkdv_kernel: a workgroup pins 128 keys (4 waves x 32) with K^T and V^T
//      in registers (V in LDS at d = 128) and streams Q, dO, LSE and -D in tiles of
//      32 query rows:
//        S = Q K^T, dP - D = dO V^T - D        (MFMA, Q and dO rows from LDS; the
//                                               accumulator starts from -D)
//        P, dS as above, per query row          (VALU)
//        dV^T += dO^T P, dK^T += Q^T dS        (MFMA, dO^T and Q^T by transposing reads)
// Fragment layouts, LDS swizzle and the key/query permutation inside each 16-wide
// MFMA step are those of the forward kernels.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const short* q;
  const short* k;
  const short* v;
  const short* o;
  const short* dout;
  const float* lse;
  float* nd;            // -D = -rowsum(dO * O), [slices_q][Nq] (workspace)
  float* l2;            // LSE in log2 units, +inf for a row that sees no key, [slices_q][Nq] (workspace)
  short* dq;
  short* dk;
  short* dv;
  int Nq, Nk;           // query rows, key rows per slice
  int Hq, group;        // query heads; query heads per K/V head (head h reads K/V head h / group)
  int off;              // causal: key j is visible to query i iff j <= i + off (off = Nk - Nq)
  int slices_q;         // B * Hq (q, o, dout, dq, lse, D are [B, Hq, Nq, ...])
  uint32_t q_bytes;     // Nq * d * 2: one query slice
  uint32_t k_bytes;     // Nk * d * 2: one K/V slice
  int qblocks, kblocks; // ceil(Nq / 128), ceil(Nk / 128)
  int dq_wgs;           // slices_q * qblocks
  int dkdv_wgs;         // B * Hk * kblocks
  float c;              // scale * log2(e)
  float scale;
};

template <bool BF16>
__device__ __forceinline__ float to_f32(short x) {
  if constexpr (BF16) return __builtin_bit_cast(float, (uint32_t)(uint16_t)x << 16);
  else return (float)__builtin_bit_cast(_Float16, x);
}

// ---- 1. D_i = dO_i . O_i -------------------------------------------------------------
// D / 8 lanes per row, 8 elements (16 bytes) each, then a butterfly sum.
// Work item of a workgroup out of T: slice and block of 128 rows (queries for dQ,
// keys for dK/dV). Contiguous ranges per XCD, so the blocks of one slice share an L2.
//
// Under a causal mask the blocks differ in length (dQ: the last query blocks see
// the most keys; dK/dV: the first key blocks are seen by the most queries). Then all
// slices' longest blocks go first, slice index fastest: with the slice count a
// multiple of 8 each XCD (blockIdx mod 8) keeps a fixed eighth of the slices and
// runs their blocks longest first. HEAVY_LAST: the longest block is the last one, so
// rank r gets block nblocks - 1 - r (dQ); otherwise block r (dK/dV). For dQ this is
// 2-4.5% faster than shortest first on the causal backward workloads (measured).
template <bool CAUSAL, bool HEAVY_LAST>
__device__ __forceinline__ void bwd_item(int T, int nblocks, int& bh, int& blk) {
  const int bid = blockIdx.x;
  if (CAUSAL) {
    const int slices = T / nblocks;
    const int rank = bid / slices;
    bh = bid - rank * slices;
    blk = HEAVY_LAST ? nblocks - 1 - rank : rank;
    return;
  }
  const int xcd = bid & 7, slot = bid >> 3, per = T >> 3, rem = T & 7;
  const int w = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  bh = w / nblocks;
  blk = w - bh * nblocks;
}

// Under a causal mask at d = 64 both kernels issue a tile's last MFMA block (dQ; dV
// and dK) at raised wave priority, so that the SIMD's other waves get the VALU for their
// weights meanwhile (whole backward, interleaved A/B: +3.4% to +4.7% on three causal
// shapes; without a mask -2.2% to +0.5%, and at d = 128 -0.6% to +0.4%, so not there;
// raising it for the first block too was slower everywhere).
template <int D, bool CAUSAL>
constexpr bool kRaiseLastBlock = D == 64 && CAUSAL;

// floor(a / b) for b > 0 and any sign of a
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Per-lane LDS element offsets of the fragment reads, for a tile of rows of D
// elements stored with swz: rowf[ks] reads 8 elements of row l32, chunk 2 ks + hi
// (an A operand row fragment); trf[db][sec] points the transposing read (see
// ds_read_tr16) so that lane i of a 16-lane group gets four consecutive rows of one
// column: together the A operand X^T with the row order of the B operands built
// from an accumulator.
template <int D, bool BYTES = false>
__device__ __forceinline__ void frag_offsets(int lane, int (&rowf)[D / 16], int (&trf)[D / 32][2]) {
  constexpr int U = BYTES ? 2 : 1;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) rowf[ks] = U * (l32 * D + (((2 * ks + hi) ^ swz<D>(l32)) << 3));
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int sec = 0; sec < 2; ++sec) {
      const int r = 4 * hi + ((lane & 15) >> 2) + 8 * sec;
      const int ch = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      trf[db][sec] = U * (r * D + ((ch ^ swz<D>(r)) << 3) + 4 * (lane & 1));
    }
}

// The element of an LDS tile at an offset in elements, or in bytes (BYTES)
template <class T, bool BYTES>
__device__ __forceinline__ const T& lds_at(const short* base, int off) {
  if constexpr (BYTES) return *(const T*)((const char*)base + off);
  else return *(const T*)(base + off);
}
// Offsets that pass through an empty asm once per tile: the compiler can no longer
// hoist offset + stage address out of the loop, and each stage's address folds into
// the reads' offset field instead of holding registers of its own. Not volatile, so
// that the asm does not split the scheduling region.
template <int D>
__device__ __forceinline__ void opaque_offsets(int (&rowf)[D / 16], int (&trf)[D / 32][2]) {
#pragma unroll
  for (int i = 0; i < D / 16; ++i) asm("" : "+v"(rowf[i]));
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) asm("" : "+v"(trf[i][h]));
}

// Direct-to-LDS loads of a 32-row tile of D columns, split over 4 waves: load i of
// the tile fills LDS bytes [1024 i, 1024 i + 1024); lane l writes tile row
// ROWS i + 16 l / (2D), chunk position (16 l mod 2D) / 16, and so fetches chunk
// position ^ swz(row) of the source row.
template <int D>
struct TileLoader {
  static constexpr int LOADS = 32 * D * 2 / 1024;   // per tile
  static constexpr int PER_WAVE = LOADS / 4;
  static constexpr int ROWS = 1024 / (2 * D);       // tile rows per load
  uint32_t off[PER_WAVE];
  int wave;
  __device__ __forceinline__ void init(int wave_, int lane) {
    wave = wave_;
#pragma unroll
    for (int kk = 0; kk < PER_WAVE; ++kk) {
      const int i = kk * 4 + wave;
      const int r_local = (16 * lane) / (2 * D);
      const int pch = ((16 * lane) % (2 * D)) / 16;
      const int r = ROWS * (i % (16 / ROWS)) + r_local;
      off[kk] = (uint32_t)((r_local * D + ((pch ^ swz<D>(r)) << 3)) * 2);
    }
  }
  // rows row0 .. row0 + 31 of the slice behind rsrc into dst
  __device__ __forceinline__ void issue(const __amdgpu_buffer_rsrc_t& rsrc, short* dst, int row0) const {
#pragma unroll
    for (int kk = 0; kk < PER_WAVE; ++kk) {
      const int i = kk * 4 + wave;
      buffer_load16_to_lds(rsrc, dst + 512 * i, off[kk], (uint32_t)((row0 + ROWS * i) * D * 2));
    }
  }
};

// 4 bytes per lane from memory into LDS: lane l writes [lds + 4 l, lds + 4 l + 4).
__device__ __forceinline__ void buffer_load4_to_lds(__amdgpu_buffer_rsrc_t r, float* lds, uint32_t voff,
                                                    uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)lds), 4, voff, soff,
      0, 0);
}

template <bool BF16>
__device__ __forceinline__ i16x8 pack8(const float (&e)[8]) {
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  e16x2 h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = __builtin_convertvector((f32x2){e[2 * i], e[2 * i + 1]}, e16x2);
  return __builtin_bit_cast(i16x8, ((u32x4){__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                            __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])}));
}

// Store a transposed accumulator: acc[db][4 g + e] of lane (hi, l32) holds
// X^T[d = 32 db + 8 g + 4 hi + e][row l32]; writes f * X[row][...] as 16-bit, 8 bytes per
// store.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows_t(short* row_ptr, int hi, const f32x16 (&acc)[D / 32], float f) {
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const e16x2 lo = __builtin_convertvector((f32x2){acc[db][4 * g] * f, acc[db][4 * g + 1] * f}, e16x2);
      const e16x2 up = __builtin_convertvector((f32x2){acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f}, e16x2);
      *(u32x2*)(row_ptr + db * 32 + 8 * g + 4 * hi) = (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, up)};
    }
}

// ---- 2. dQ -----------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dq_kernel(BwdParams p) {
#pragma clang fp contract(off)
  constexpr int BM = 128, BN = 32, TILE = BN * D;
  __shared__ __attribute__((aligned(1024))) short lds_k0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_k1[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v1[TILE];

  int bh, blk;
  bwd_item<CAUSAL, true>(p.dq_wgs, p.qblocks, bh, blk);   // causal: the last (longest) query blocks first
  const int Nq = p.Nq, Nk = p.Nk, off = p.off;
  const int m0 = blk * BM;
  const int b = bh / p.Hq, h = bh - b * p.Hq;
  const int64_t base = (int64_t)bh * Nq * D;                                       // query slice
  const int64_t base_k = ((int64_t)b * (p.Hq / p.group) + h / p.group) * Nk * D;  // its K/V slice
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + base, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base_k, p.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base_k, p.k_bytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wq0 = m0 + 32 * wave;
  const int qrow = wq0 + l32;
  const float c = p.c;

  int rowf[D / 16], trf[D / 32][2];
  frag_offsets<D>(lane, rowf, trf);
  TileLoader<D> ld;
  ld.init(wave, lane);

  // Q^T and dO^T as B operands: 8 consecutive columns of this lane's query row
  i16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = buffer_load16(rq, (uint32_t)((qrow * D + ks * 16 + 8 * hi) * 2));
    dof[ks] = buffer_load16(rdo, (uint32_t)((qrow * D + ks * 16 + 8 * hi) * 2));
  }
  // This lane's query: D = dO . O, the row sum that dS = P (dP - D) needs, and the
  // LSE in log2 units (+inf, i.e. no weight, for a row that sees no key or lies past
  // Nq). Lanes l32 and l32 + 32 hold the row's columns 16 ks + 8 hi .. +7: each sums
  // its own and the two halves are added. Both values also go to the workspace for
  // the dK/dV kernel, which runs after this one on the same stream.
  const bool live = qrow < Nq;
  float dpart = 0.f;
  {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + base, p.q_bytes);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const i16x8 of = buffer_load16(ro, (uint32_t)((qrow * D + ks * 16 + 8 * hi) * 2));
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf(to_f32<BF16>(dof[ks][e]), to_f32<BF16>(of[e]), dpart);
    }
  }
  const float dsum = sum_halves(dpart);
  const float lse_nat = live ? p.lse[(int64_t)bh * Nq + qrow] : -INFINITY;
  const float lse2 = lse_nat == -INFINITY ? INFINITY : lse_nat * kLog2e;
  const float dl = live ? dsum : 0.f;
  if (live && hi == 0) {
    p.nd[(int64_t)bh * Nq + qrow] = -dsum;
    p.l2[(int64_t)bh * Nq + qrow] = lse2;
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // The dP accumulation starts from -D (a block of 16 registers that stays for the
  // whole loop, the C operand of each tile's first dP MFMA), so that the MFMAs yield
  // dP - D and dS = P (dP - D) is one multiply per score (measured: the backward
  // +1.4% to +2.6% at d = 64, +0.8% at d = 128). At d = 128 under the causal mask those
  // 16 registers do not fit, and dS takes a subtraction as well.
  constexpr bool DP_MINUS_D = D == 64 || !CAUSAL;
  f32x16 dp0;
#pragma unroll
  for (int r = 0; r < 16; ++r) dp0[r] = DP_MINUS_D ? -dl : 0.f;

  const int n_end = CAUSAL ? max(0, min(Nk, m0 + BM + off)) : Nk;
  const int ntiles = (n_end + BN - 1) / BN;

  auto sync_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };

  // One key tile: K rows in kbuf, V rows in vbuf (this iteration's stage); `mask` is a
  // wave-uniform flag. (A second copy of this code without the mask, chosen at compile
  // time, paid while a masked score cost about five instructions; with the one-compare
  // mask the single copy is 5-7% faster at d = 64, measured, and needs fewer registers.)
  auto step = [&](int n0, const short* kbuf, const short* vbuf, bool mask) __attribute__((always_inline)) {
    f32x16 s, dp;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const i16x8 a = *(const i16x8*)(kbuf + rowf[ks]);
      const i16x8 b = *(const i16x8*)(vbuf + rowf[ks]);
      s = mfma_32x32x16<BF16>(a, qf[ks], ks == 0 ? f32x16{} : s);
      dp = mfma_32x32x16<BF16>(b, dof[ks], ks == 0 ? dp0 : dp);
    }
    // s[r], dp[r]: key n0 + 8 (r / 4) + 4 hi + r % 4, query qrow
    // The mask is applied to the whole tile behind one wave-uniform branch: a block
    // this size is not speculated into per-score selects on the unmasked tiles.
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
    if (mask) {
      // hidden: key >= Nk or (causal) key > qrow + off, i.e. key > min(Nk - 1, qrow + off);
      // one compare per score against the lane's limit
      const int lim = (CAUSAL ? min(Nk - 1, qrow + off) : Nk - 1) - (n0 + 4 * hi);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) > lim) pr[r] = 0.f;
    }
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) ds[r] = DP_MINUS_D ? pr[r] * dp[r] : pr[r] * (dp[r] - dl);
    i16x8 dsp[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = ds[8 * tt + i];
      dsp[tt] = pack8<BF16>(e);
    }
    // dQ^T += K^T dS^T
    if constexpr (kRaiseLastBlock<D, CAUSAL>) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const short* src = kbuf + 16 * tt * D;
        const i16x4 a0 = ds_read_tr16(src + trf[db][0]);
        const i16x4 a1 = ds_read_tr16(src + trf[db][1]);
        acc[db] = mfma_32x32x16<BF16>(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), dsp[tt], acc[db]);
      }
    if constexpr (kRaiseLastBlock<D, CAUSAL>) __builtin_amdgcn_s_setprio(0);
  };

  auto tile = [&](int j, short* k_rd, short* v_rd, short* k_wr, short* v_wr) __attribute__((always_inline)) {
    sync_tile();
    if (j + 1 < ntiles) {
      ld.issue(rk, k_wr, (j + 1) * BN);
      ld.issue(rv, v_wr, (j + 1) * BN);
    }
    const int n0 = j * BN;
    if (CAUSAL && n0 > wq0 + 31 + off) return;   // whole tile in this wave's future
    // a tile needs the mask if it reaches past Nk or, under a causal mask, past the
    // diagonal of this wave's first query (decided per wave, not per workgroup)
    step(n0, k_rd, v_rd, n0 + BN > Nk || (CAUSAL && n0 + BN - 1 > wq0 + off));
  };
  if (ntiles > 0) {
    ld.issue(rk, lds_k0, 0);
    ld.issue(rv, lds_v0, 0);
  }
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    tile(j, lds_k0, lds_v0, lds_k1, lds_v1);
    tile(j + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }
  if (j < ntiles) tile(j, lds_k0, lds_v0, lds_k1, lds_v1);

  if (live) store_rows_t<D, BF16>(p.dq + base + (int64_t)qrow * D, hi, acc, p.scale);
}

// ---- 3. dK and dV --------------------------------------------------------------------
// At d = 128, K^T and V^T fragments in registers plus both accumulators need more
// than 256 registers. So the workgroup's V rows stay in LDS (32 KB), the V^T
// fragments are read per tile and the LDS fragment offsets are recomputed per tile:
// two waves per SIMD without spills (228 VGPRs, 253 under the causal mask).
// Measured against one wave per SIMD with everything in registers: 22% faster
// without a mask, 21% faster with one.
template <int D, bool BF16, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fa_bwd_dkdv_kernel(BwdParams p) {
#pragma clang fp contract(off)
  constexpr int BK = 128, BQ = 32, TILE = BQ * D;
  constexpr bool V_LDS = D == 128;
  __shared__ __attribute__((aligned(1024))) short lds_vk[V_LDS ? BK * D : 8];
  __shared__ __attribute__((aligned(1024))) short lds_q0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_q1[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_o0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_o1[TILE];
  __shared__ __attribute__((aligned(256))) float lds_l0[64];
  __shared__ __attribute__((aligned(256))) float lds_l1[64];
  __shared__ __attribute__((aligned(256))) float lds_d0[64];
  __shared__ __attribute__((aligned(256))) float lds_d1[64];

  int bhk, blk;                                 // K/V slice (batch, K/V head) and key block
  bwd_item<CAUSAL, false>(p.dkdv_wgs, p.kblocks, bhk, blk);
  const int Nq = p.Nq, Nk = p.Nk, off = p.off, group = p.group;
  const int hk_count = p.Hq / group;
  const int b = bhk / hk_count, kh = bhk - b * hk_count;
  const int n0 = blk * BK;                      // first key of this workgroup
  const int64_t base = (int64_t)bhk * Nk * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base, p.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base, p.k_bytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int k0 = n0 + 32 * wave;                // this wave's first key
  const int key = k0 + l32;                     // this lane's key (column of S, dP)
  const int key_rel = key - off;                // visible to query i iff key_rel <= i
  const float c = p.c;

  // Fragment offsets: see the step below.
  constexpr bool OPQ = V_LDS && !CAUSAL;
  int rowf[D / 16], trf[D / 32][2];
  frag_offsets<D, OPQ>(lane, rowf, trf);
  TileLoader<D> ld;
  ld.init(wave, lane);

  // K^T and V^T as B operands: 8 consecutive columns of this lane's key row (V^T
  // from LDS per tile when V_LDS)
  i16x8 kf[D / 16], vf[V_LDS ? 1 : D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kf[ks] = buffer_load16(rk, (uint32_t)((key * D + ks * 16 + 8 * hi) * 2));
  if constexpr (V_LDS) {
#pragma unroll
    for (int b = 0; b < BK / BQ; ++b) ld.issue(rv, lds_vk + b * BQ * D, n0 + b * BQ);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) vf[ks] = buffer_load16(rv, (uint32_t)((key * D + ks * 16 + 8 * hi) * 2));
  }
  const short* vrows = lds_vk + 32 * wave * D;   // this wave's 32 V rows (V_LDS)
  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) { adk[db][r] = 0.f; adv[db][r] = 0.f; }

  // Query tiles of 32 rows, for each of the group's query heads in turn. Under a
  // causal mask a tile matters once its
  // last query sees a key of this workgroup (32 t + 31 + off >= n0), and for a wave
  // once it sees one of the wave's keys; the wave's tiles up to the one whose first
  // query sees its last key need the mask.
  const int T = (Nq + BQ - 1) / BQ;
  const int t0 = CAUSAL ? max(0, -floor_div(off + 31 - n0, BQ)) : 0;
  const int t_wave = CAUSAL ? max(0, -floor_div(off + 31 - k0, BQ)) : 0;
  const int t_nomask = CAUSAL ? -floor_div(off - 31 - k0, BQ) : 0;    // tiles from here need no causal mask

  // buffer descriptors of the query head being processed
  __amdgpu_buffer_rsrc_t rq, rdo, rls, rdl;
  auto set_head = [&](int g) __attribute__((always_inline)) {
    const int64_t bq = (int64_t)b * p.Hq + kh * group + g;   // query slice
    rq = make_rsrc(p.q + bq * Nq * D, p.q_bytes);
    rdo = make_rsrc(p.dout + bq * Nq * D, p.q_bytes);
    rls = make_rsrc(p.l2 + bq * Nq, (uint32_t)Nq * 4);
    rdl = make_rsrc(p.nd + bq * Nq, (uint32_t)Nq * 4);
  };
  auto issue = [&](int t, short* qd, short* od, float* lsd, float* dd) __attribute__((always_inline)) {
    ld.issue(rq, qd, t * BQ);
    ld.issue(rdo, od, t * BQ);
    if (wave == 0) buffer_load4_to_lds(rls, lsd, (uint32_t)(4 * lane), (uint32_t)(t * BQ * 4));
    if (wave == 1) buffer_load4_to_lds(rdl, dd, (uint32_t)(4 * lane), (uint32_t)(t * BQ * 4));
  };
  auto sync_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };

  // Score r of query tile t belongs to query t BQ + 4 hi + q_r, q_r = 8 (r / 4) + r % 4.
  // It is hidden when the query is past Nq or (causal) before this lane's key_rel:
  // two compares of q_r against the lane's limits.
  struct MaskLimits {
    int last, first;   // visible iff first <= q_r <= last
    __device__ bool hidden(int q_r) const { return q_r > last || (CAUSAL && q_r < first); }
  };
  auto mask_limits = [&](int t) __attribute__((always_inline)) {
    const int q0 = t * BQ + 4 * hi;
    return MaskLimits{Nq - 1 - q0, key_rel - q0};
  };
  // `mask`: a wave-uniform flag, as in the dQ kernel
  auto step = [&](int t, const short* qbuf, const short* obuf, const float* lsb, const float* db_, bool mask)
      __attribute__((always_inline)) {
    // With V in LDS the registers are the scarce resource. Without a mask the
    // offsets pass through opaque_offsets, which keeps them from multiplying by the
    // LDS stages (+3.6% to +3.9% for the whole backward at d = 128 against the per-tile
    // recomputation); under the causal mask that still spills, and the offsets are
    // recomputed per tile from the lane index (one XOR-shift each) instead of staying
    // live across the loop.
    constexpr bool RECOMP = V_LDS && !OPQ;
    int rfv[D / 16], tfv[D / 32][2];
    if constexpr (OPQ) opaque_offsets<D>(rowf, trf);
    if constexpr (RECOMP) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      frag_offsets<D>(ln, rfv, tfv);
    }
    const int(&rf)[D / 16] = RECOMP ? rfv : rowf;
    const int(&tf)[D / 32][2] = RECOMP ? tfv : trf;
    // dP starts from -D of its query rows, so the products land as dP - D
    f32x16 s, dp;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const f32x4 nd4 = *(const f32x4*)(db_ + 8 * g + 4 * hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) { s[4 * g + e] = 0.f; dp[4 * g + e] = nd4[e]; }
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) s = mfma_32x32x16<BF16>(lds_at<i16x8, OPQ>(qbuf, rf[ks]), kf[ks], s);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const i16x8 b = lds_at<i16x8, OPQ>(obuf, rf[ks]);
      i16x8 vk;
      if constexpr (V_LDS) vk = lds_at<i16x8, OPQ>(vrows, rf[ks]);
      else vk = vf[ks];
      dp = mfma_32x32x16<BF16>(b, vk, dp);
    }
    // s[r], dp[r]: query t BQ + 8 (r / 4) + 4 hi + r % 4, key `key`.
    i16x8 pp[2], dsp[2];
    if constexpr (D == 64) {
      // The mask is applied to the whole tile behind one wave-uniform branch (a block
      // this size is not speculated into per-score selects on the unmasked tiles).
      float w[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 l4 = *(const f32x4*)(lsb + 8 * g + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * g + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c, -l4[e]));
      }
      if (mask) {
        const MaskLimits ml = mask_limits(t);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (ml.hidden(8 * (r >> 2) + (r & 3))) w[r] = 0.f;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e1[8], e2[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e1[i] = w[8 * tt + i];
          e2[i] = w[8 * tt + i] * dp[8 * tt + i];
        }
        pp[tt] = pack8<BF16>(e1);
        dsp[tt] = pack8<BF16>(e2);
      }
    } else {
      // At d = 128 the sixteen weights of the tile cannot all stay live (the kernel
      // spills): each half (8 rows) is formed, masked behind one wave-uniform branch,
      // rounded and packed in turn.
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e1[8], e2[8];
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const int g = 2 * tt + gg;
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          const f32x4 l4 = *(const f32x4*)(lsb + 8 * g + 4 * hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) e1[4 * gg + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c, -l4[e]));
        }
        if (mask) {
          const MaskLimits ml = mask_limits(t);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (ml.hidden(8 * (2 * tt + (i >> 2)) + (i & 3))) e1[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) e2[i] = e1[i] * dp[8 * tt + i];
        pp[tt] = pack8<BF16>(e1);
        dsp[tt] = pack8<BF16>(e2);
      }
    }
    // dV^T += dO^T P, dK^T += Q^T dS
    if constexpr (kRaiseLastBlock<D, CAUSAL>) __builtin_amdgcn_s_setprio(2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i16x4 o0 = ds_read_tr16(&lds_at<short, OPQ>(obuf + 16 * tt * D, tf[db][0]));
        const i16x4 o1 = ds_read_tr16(&lds_at<short, OPQ>(obuf + 16 * tt * D, tf[db][1]));
        const i16x4 q0 = ds_read_tr16(&lds_at<short, OPQ>(qbuf + 16 * tt * D, tf[db][0]));
        const i16x4 q1 = ds_read_tr16(&lds_at<short, OPQ>(qbuf + 16 * tt * D, tf[db][1]));
        adv[db] = mfma_32x32x16<BF16>(__builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7), pp[tt], adv[db]);
        adk[db] = mfma_32x32x16<BF16>(__builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7), dsp[tt], adk[db]);
      }
    if constexpr (kRaiseLastBlock<D, CAUSAL>) __builtin_amdgcn_s_setprio(0);
  };

  auto tile = [&](int t, short* q_rd, short* o_rd, float* l_rd, float* d_rd, short* q_wr, short* o_wr, float* l_wr,
                  float* d_wr) __attribute__((always_inline)) {
    sync_tile();
    if (t + 1 < T) issue(t + 1, q_wr, o_wr, l_wr, d_wr);
    if (t < t_wave) return;                       // no query of this tile sees this wave's keys
    step(t, q_rd, o_rd, l_rd, d_rd, (CAUSAL && t < t_nomask) || (t + 1) * BQ > Nq);
  };
  // The query heads that share this K/V head, one after the other (one head without
  // grouping). Loads are double-buffered within a head; a new head starts once every
  // wave is done with the previous head's last tile.
  for (int g = 0; g < group; ++g) {
    if (g > 0) __syncthreads();
    set_head(g);
    if (t0 < T) issue(t0, lds_q0, lds_o0, lds_l0, lds_d0);
    int t = t0;
    for (; t + 1 < T; t += 2) {
      tile(t, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);
      tile(t + 1, lds_q1, lds_o1, lds_l1, lds_d1, lds_q0, lds_o0, lds_l0, lds_d0);
    }
    if (t < T) tile(t, lds_q0, lds_o0, lds_l0, lds_d0, lds_q1, lds_o1, lds_l1, lds_d1);
  }

  if (key < Nk) {
    store_rows_t<D, BF16>(p.dk + base + (int64_t)key * D, hi, adk, p.scale);
    store_rows_t<D, BF16>(p.dv + base + (int64_t)key * D, hi, adv, 1.f);
  }
}

template <int D, bool BF16>
hipError_t launch_bwd(const BwdParams& p, bool causal, hipStream_t s) {
  // The dQ kernel writes -D and the base-2 LSE of every query row before the dK/dV
  // kernel reads them (stream order). dq_wgs is 0 only without query rows, dkdv_wgs
  // only without keys.
  hipError_t e = hipSuccess;
  if (causal) {
    if (p.dq_wgs > 0) e = launch_kernel(&fa_bwd_dq_kernel<D, BF16, true>, p.dq_wgs, 256, s, p);
    if (e == hipSuccess && p.dkdv_wgs > 0) e = launch_kernel(&fa_bwd_dkdv_kernel<D, BF16, true>, p.dkdv_wgs, 256, s, p);
  } else {
    if (p.dq_wgs > 0) e = launch_kernel(&fa_bwd_dq_kernel<D, BF16, false>, p.dq_wgs, 256, s, p);
    if (e == hipSuccess && p.dkdv_wgs > 0) e = launch_kernel(&fa_bwd_dkdv_kernel<D, BF16, false>, p.dkdv_wgs, 256, s, p);
  }
  return e;
}

// Shared by fa_bwd and fa_bwd_ex: contiguous [B, H, N, d] tensors, K/V heads shared by
// Hq / Hk query heads, Nq queries against Nk keys (causal: bottom-right alignment).
fa_status run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d,
                  float scale, int causal, fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || Hq < 0 || Hk < 0 || Nq < 0 || Nk < 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_BAD_DTYPE;
  if (B == 0 || (Hq == 0 && Hk == 0)) return FA_OK;
  if (Hq == 0 || Hk == 0 || Hq % Hk != 0) return FA_ERR_BAD_SHAPE;
  if (Nq == 0 && Nk == 0) return FA_OK;
  const bool has_q = Nq > 0, has_k = Nk > 0;
  if ((has_q && (!q || !o || !dout || !lse || !dq)) || (has_k && (!k || !v || !dk || !dv))) return FA_ERR_NULL_PTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return FA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;
  // one slice plus the padded last block in 32-bit byte offsets; grid and row counts in int
  if ((Nq + 512) * d * 2 >= ((int64_t)1 << 31) || (Nk + 512) * d * 2 >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  const int64_t qblocks = (Nq + 127) / 128, kblocks = (Nk + 127) / 128;
  if (B * Hq >= ((int64_t)1 << 31) / (qblocks + kblocks + 1)) return FA_ERR_TOO_LARGE;
  if (B * Hq * Nq >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  if (has_q && (!workspace || ((uintptr_t)workspace & 15) || workspace_bytes < (size_t)(B * Hq * Nq) * 8))
    return FA_ERR_WORKSPACE;
  BwdParams p;
  p.q = (const short*)q;
  p.k = (const short*)k;
  p.v = (const short*)v;
  p.o = (const short*)o;
  p.dout = (const short*)dout;
  p.lse = lse;
  p.nd = (float*)workspace;
  p.l2 = (float*)workspace + B * Hq * Nq;
  p.dq = (short*)dq;
  p.dk = (short*)dk;
  p.dv = (short*)dv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.Hq = (int)Hq;
  p.group = (int)(Hq / Hk);
  p.off = (int)(Nk - Nq);
  p.slices_q = (int)(B * Hq);
  p.q_bytes = (uint32_t)(Nq * d * 2);
  p.k_bytes = (uint32_t)(Nk * d * 2);
  p.qblocks = (int)qblocks;
  p.kblocks = (int)kblocks;
  p.dq_wgs = (int)(B * Hq * qblocks);
  p.dkdv_wgs = (int)(B * Hk * kblocks);
  p.c = (float)((double)scale * 1.4426950408889634);
  p.scale = scale;
  const hipStream_t s = stream;
  const bool bf16 = dtype == FA_BF16;
  hipError_t e;
  if (d == 64) e = bf16 ? launch_bwd<64, true>(p, causal != 0, s) : launch_bwd<64, false>(p, causal != 0, s);
  else e = bf16 ? launch_bwd<128, true>(p, causal != 0, s) : launch_bwd<128, false>(p, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)(B * H * N) * 8;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                 fa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, N, d, scale, causal, dtype, workspace,
                 workspace_bytes, stream);
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk,
                    int64_t d, float scale, int causal, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, Hq, Hk, Nq, Nk, d, scale, causal, dtype, workspace,
                 workspace_bytes, stream);
}

}  // extern "C"
