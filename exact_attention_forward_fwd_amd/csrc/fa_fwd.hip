// Exact attention forward (FlashAttention-2 loop order) for MI355X / gfx950 (CDNA4).
//
// One workgroup owns BM query rows of one (batch, head) slice; each of its waves owns
// 32 or 64 of them (one or two 32-query blocks). The workgroup streams K and V in
// tiles of BN keys, straight from memory into double-buffered LDS. Per tile, every wave
//   1. computes S^T = K_tile Q_w^T on v_mfma_f32_32x32x16_{f16,bf16} (fp32 acc):
//      with the keys as MFMA rows and the queries as columns, each lane ends up
//      holding one query's scores for 16 keys of every 32-key block, so the
//      row (per-query) reductions are in-lane ops plus one permlane32 swap;
//   2. masks the causal diagonal / ragged tail to -inf (only on tiles that need it);
//   3. updates the online-softmax state in registers. The weights are formed against
//      the current exponent reference, P = 2^(c x - ref) with c = s log2(e) folded
//      into one FMA, and their per-lane sum both updates l and checks the reference:
//      while it stays at most 2^8, so does every weight. On a row's first tile, or
//      when a sum exceeds 2^8 (a new maximum well above the reference), the tile is
//      redone after moving the reference up to the row maximum, ref = fl(c m), and
//      rescaling l and U by alpha = 2^(ref_old - ref_new). No row maximum is needed
//      on the common path;
//   4. rounds P to 16 bits in registers; those registers are directly the B
//      operand of O^T += V^T P^T (the key order inside each 16-key MFMA step is
//      permuted identically on both operands, which a sum over keys allows), issued
//      one tile later so that these MFMAs overlap the next tile's softmax;
//   5. reads V^T fragments with ds_read_b64_tr_b16 (transposing 16-bit LDS reads).
// After the last tile: O = U / l, LSE = ln2 (ref + log2 l), written once.
//
// The method is that of "用 CuTe 读懂 FlashAttention" (blog.qingsen.net): one block
// pins a Q tile and walks the K/V tiles (its opening example and step 1), the
// online-softmax state and recurrence of step 4, P kept in registers as the second
// GEMM's operand (step 5), whole-tile skipping plus element masking for causal
// (causal section) and the single final normalisation with the LSE side output
// (final section); loop order and the -inf guard follow "CUDA 算子工程" ch. 14
// §14.5. Register/LDS layout, the transposed-Q formulation, the deferred P V and the
// instruction choices are this file's own, made for CDNA4's 64-wide waves and MFMA shapes.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <mutex>
#include <type_traits>

#include "fa.h"
#include "fa_device.h"

// This file is compiled twice (build.py), with different instruction schedulers: as
// a whole, and with FA_FWD_DEFAULT_SCHED_UNIT defined, when it holds only the launches
// of the four-wave kernel under a causal mask and of its two-wave tiles (the kernels
// that the maximum-ILP schedule slows down). The launch parameters cross between the
// two units, so they live in a named namespace.
namespace fa_fwd_unit {

// One launch: B batches of Hq query heads; query head h reads K/V head h / group.
// Tensors are [B, heads, rows, d] with arbitrary batch/head/row strides (elements)
// and contiguous d; LSE is [B, Hq, Nq] contiguous.
struct Params {
  const short* q;
  const short* k;
  const short* v;
  short* o;
  float* lse;
  int Nq, Nk;         // query rows, key rows per slice
  int Hq;             // query heads
  int group;          // query heads per K/V head
  int causal_off;     // causal: key j is valid for query i iff j <= i + causal_off
  int qmod;           // 0: row r of a slice is query r; > 0: the query heads of a group
                      // are packed into one slice and row r is query r mod qmod
  int q_sr, k_sr, v_sr, o_sr;                      // row strides
  int64_t q_sb, q_sh, k_sb, k_sh, v_sb, v_sh, o_sb, o_sh;   // batch and head strides
  uint32_t q_bytes, k_bytes, v_bytes;              // extent of one slice: rows past it read as zeros
  int num_m_blocks;   // ceil(Nq / BM)
  int num_splits;     // key ranges per query block (split-KV); 1: all keys in one workgroup
  int split_keys;     // keys per range, a multiple of the key tile
  int slices;         // B * Hq
  int total_wgs;      // slices * num_splits * num_m_blocks
  float c;            // scale * log2(e)
  // Split-KV partial results, or null: O_k = U_k / l_k as fp32 [num_splits][slices][Nq][d]
  // and LSE_k as [num_splits][slices][Nq], in place of o and lse.
  float* po;
  float* plse;
};

// Launch of fa_fwd_kernel<d, bf16, causal, nw, qb, bn> from the unit built with the
// default scheduler; causal or nw == 2 only.
hipError_t launch_default_sched(const Params& p, int d, bool bf16, bool causal, int nw, int bn, int qb,
                                hipStream_t stream);

}  // namespace fa_fwd_unit

namespace {

using fa_fwd_unit::Params;

// Work item of a workgroup: slice (batch, query head), key range and query block.
// The workgroups of one XCD take a contiguous range of items (dispatch is
// round-robin over the 8 XCDs), so the query blocks that stream the same K and V
// share that XCD's L2. Under a causal mask the longest query blocks go first.
struct WorkItem { int bh, split, mb; };
template <bool CAUSAL, int GROUP = 0>
__device__ __forceinline__ WorkItem work_item(const Params& p) {
  const int bid = blockIdx.x;
  const int T = p.total_wgs;
  if (CAUSAL) {
    // Causal row blocks differ in length (block mb sees mb + 1 blocks of keys): all
    // slices' longest blocks first, slice index fastest. Workgroup b runs on XCD b mod
    // 8, so with the slice count a multiple of 8 each XCD keeps a fixed eighth of the
    // slices and runs their blocks longest first. Measured against slice-contiguous
    // ranges per XCD: +17% (n2048 d128), +25% (n1000 d64), +26% (n4096 d64); +10% to
    // +23% with 12 or 36 slices, where a slice's blocks spread over the XCDs.
    const int slices = T / (p.num_m_blocks * p.num_splits);
    if (GROUP > 0 && slices % (8 * GROUP) == 0) {
      // The same per-XCD slices (bh = 8 ls + XCD), taken GROUP at a time, longest
      // blocks first within each group, so that more of an XCD's resident workgroups
      // stream the same K/V. Measured with the pipelined kernel (GROUP = 8, sustained
      // back-to-back timing): +0.3% to +4.7% on seven causal d = 128 shapes (N = 1024
      // to 4096, 32 to 128 slices); with the four-wave kernel at d = 64, -4.1% to +3.1%,
      // so it keeps the plain order.
      const int xcd = bid & 7, k = bid >> 3;
      const int per_group = GROUP * p.num_m_blocks * p.num_splits;
      const int g = k / per_group, r = k - g * per_group;
      const int rank = r / GROUP, sg = r - rank * GROUP;
      const int mb_rank = rank / p.num_splits, split = rank - mb_rank * p.num_splits;
      return {(g * GROUP + sg) * 8 + xcd, split, p.num_m_blocks - 1 - mb_rank};
    }
    const int rank = bid / slices, bh = bid - rank * slices;
    const int mb_rank = rank / p.num_splits, split = rank - mb_rank * p.num_splits;
    return {bh, split, p.num_m_blocks - 1 - mb_rank};
  }
  const int xcd = bid & 7, slot = bid >> 3, per = T >> 3, rem = T & 7;
  const int w = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int per_slice = p.num_m_blocks * p.num_splits;
  const int bh = w / per_slice;
  const int r = w - bh * per_slice;
  const int split = r / p.num_m_blocks;
  return {bh, split, r - split * p.num_m_blocks};
}

// Base pointers of one (batch, query head) slice and of the K/V head it reads.
struct Slice {
  const short* q;
  const short* k;
  const short* v;
  short* o;
};
__device__ __forceinline__ Slice slice_of(const Params& p, int bh) {
  const int b = bh / p.Hq, h = bh - b * p.Hq, kh = h / p.group;
  return {p.q + b * p.q_sb + h * p.q_sh, p.k + b * p.k_sb + kh * p.k_sh, p.v + b * p.v_sb + kh * p.v_sh,
          p.o + b * p.o_sb + h * p.o_sh};
}


// The softmax keeps its exponent reference while a lane's weights of one tile sum to
// at most this, which bounds every weight by it as well (2^8, far inside fp16's
// range). The final O = U / l and LSE = ln2 (ref + log2 l) hold for any common
// reference, so keeping it, instead of moving it on every new maximum, changes
// nothing but rounding.
constexpr float kSumMax = 256.0f;

// Row sums of fp16 weights in unmasked tiles. Each lane's sum over a tile is formed
// from the rounded weights (the values the second product multiplies): packed fp16
// adds of pairs of pairs, so that each half sums four weights, then mixed-precision
// FMAs into one fp32 sum. That is 9 instructions per 16 weights instead of 15 fp32
// adds; a wave's softmax runs at its instruction issue rate, so this is what counts
// (measured +6.5% to +7% on B=2 H=16 N=4096 d=64 and at N = 2048 and 8192 without a
// mask, +1.5% at N = 4096 under a causal mask, +0.5% at N = 1000 causal). Each weight
// is within 2^-12 of its fp32 value relative to it and each fp16 add rounds to 2^-12
// of its sum, so a tile's sum is within 3 * 2^-12 (7.3e-4) of the exact one, relative;
// O = U / l is then the exact convex combination of the rounded weights U holds, and
// LSE moves by at most that much where one tile holds a row's mass, by far less where
// many tiles share it.
// Masked tiles (the causal diagonal, the ragged end), where rows with few visible keys
// have their mass, and bf16 weights (rounded to 2^-9) keep fp32 sums of the fp32 weights.
constexpr bool kPackedSums = true;

// The P V MFMAs are issued at raised wave priority: the SIMD's other wave then gets
// the VALU for its softmax while these MFMAs stream (measured: 5-20% faster). At
// d = 64, where the softmax dominates, the four-wave kernel raises it for the whole
// MFMA section of a tile (S and P V: 2.4% faster than P V alone, measured; at
// d = 128 that was 5% slower).
constexpr bool kRaisePvPriority = true;

// Epilogue of one wave: O = U / l and LSE = ln2 (ref + log2 l) for its QB blocks of 32
// queries (l is split between the two lane halves), rounded into o and lse; or, for
// a split-KV range, the fp32 partials O_k and LSE_k. A row with no visible key
// (l = 0) gets O = 0 and LSE = -inf. acc_o[qb][db][4 g + e] of lane (hi, l32) holds
// U^T[d = 32 db + 8 g + 4 hi + e][query wq0 + 32 qb + l32].
template <int D, bool BF16, int QB>
__device__ __forceinline__ void write_rows(const Params& p, const Slice& sl, int bh, int split, int wq0, int lane,
                                           const f32x16 (&acc_o)[QB][D / 32], const float (&ref)[QB],
                                           const float (&l_run)[QB]) {
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using f32x4 = float __attribute__((ext_vector_type(4)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = wq0 + 32 * qb + l32;
    const float l_tot = sum_halves(l_run[qb]);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow >= p.Nq) continue;
    const float lse = (l_tot > 0.f) ? kLn2 * (ref[qb] + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
    if (p.po) {
      const int64_t row = ((int64_t)split * p.slices + bh) * p.Nq + qrow;
      float* prow = p.po + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4*)(prow + db * 32 + 8 * g + 4 * hi) =
              (f32x4){acc_o[qb][db][4 * g] * inv, acc_o[qb][db][4 * g + 1] * inv, acc_o[qb][db][4 * g + 2] * inv,
                      acc_o[qb][db][4 * g + 3] * inv};
      if (hi == 0) p.plse[row] = lse;
    } else {
      short* orow = sl.o + (int64_t)qrow * p.o_sr;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          e16x2 lo = __builtin_convertvector((f32x2){acc_o[qb][db][4 * g + 0] * inv, acc_o[qb][db][4 * g + 1] * inv}, e16x2);
          e16x2 up = __builtin_convertvector((f32x2){acc_o[qb][db][4 * g + 2] * inv, acc_o[qb][db][4 * g + 3] * inv}, e16x2);
          *(u32x2*)(orow + db * 32 + 8 * g + 4 * hi) =
              (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, up)};
        }
      if (hi == 0) p.lse[(int64_t)bh * p.Nq + qrow] = lse;
    }
  }
}

// Two waves per SIMD: one wave's MFMAs run while the other does its softmax. The
// register budget (<= 256 per lane) is part of the kernel's design, not a hint.
constexpr int WAVES_PER_SIMD = 2;

// NW waves per workgroup; each wave owns QB blocks of 32 queries (BM = 32 NW QB
// query rows per workgroup) and shares every K and V fragment it reads from LDS
// across those QB blocks.
//
// Pipeline (one barrier per key tile j):
//   wait for this wave's loads, barrier      K(j) and V(j-1) are in LDS
//   start loads K(j+1) -> kbuf[(j+1)%2], V(j) -> vbuf[j%2]   (LDS direct, async)
//   S = K(j) Q^T                              MFMA
//   U += V(j-1)^T P(j-1)^T                     MFMA, independent of S
//   softmax of S -> P(j), kept for the next iteration     VALU, overlaps the PV MFMAs
// The weights of tile j enter U one iteration later; a reference move (rare) first
// lets the pending P(j-1) V(j-1) land in U, then scales U and l by alpha.
template <int D, bool BF16, bool CAUSAL, int NW, int QB, int BN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD))) void fa_fwd_kernel(Params p) {
  // Every fused multiply-add below is written out; the compiler must not fuse the
  // rounded reference products into neighbouring adds (see the softmax state note).
#pragma clang fp contract(off)
  constexpr int BM = 32 * NW * QB;          // query rows per workgroup
  constexpr int TILE = BN * D;              // elements per K or V tile
  constexpr int DMA_PER_TILE = TILE * 2 / 1024;   // 1 KB direct-to-LDS loads per tensor per tile
  constexpr int DMA_PER_WAVE = DMA_PER_TILE / NW;
  constexpr int ROWS_PER_DMA = 1024 / (2 * D);    // tile rows one 1 KB load covers
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "tile shape");
  constexpr int PATS = 16 / ROWS_PER_DMA;          // loads per 16-row swizzle period
  static_assert(DMA_PER_TILE % NW == 0, "every wave issues the same number of loads");
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;

  // Two stages per tensor, as four distinct LDS objects: with the tile loop unrolled
  // by two every access names its stage at compile time, so the compiler can tell
  // the stage being read from the one the in-flight direct loads are filling and
  // does not wait for those loads before reading.
  __shared__ __attribute__((aligned(1024))) short lds_k0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_k1[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v1[TILE];

  const WorkItem wi = work_item<CAUSAL>(p);
  const int bh = wi.bh;
  const int Nk = p.Nk, off = p.causal_off;
  const int m0 = wi.mb * BM;
  // keys [kb, ke) of this workgroup's range
  const int kb = wi.split * p.split_keys;
  const int ke = min(Nk, kb + p.split_keys);
  const Slice sl = slice_of(p, bh);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(sl.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(sl.k, p.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(sl.v, p.v_bytes);

  const int tid = threadIdx.x;
  // the wave index is uniform across the wave; saying so keeps LDS-load bases and
  // buffer offsets in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wq0 = m0 + wave * 32 * QB;     // first query of this wave
  const float c = p.c;
  // 1.0 kept out of the compiler's sight, so that x * one + sum with an fp16 x stays one
  // v_fma_mix_f32 instead of a conversion and an add
  float one = 1.0f;
  asm("" : "+s"(one));

  // ---- per-lane LDS offsets (elements) ----
  // K fragment (A operand of S^T = K Q^T): row 32 kb + l32, 16-byte chunk 2 ks + hi.
  // V^T fragment via ds_read_b64_tr_b16. Lane (group of 16 = g, index i) receives
  // element j from lane 4j + i/4 of its group, component i%4. With lane L of the
  // group pointing at V[key0 + L/4][dcol0 + 4 (L%4)], lane i gets V[key0 + j][dcol0 + i],
  // j = 0..3: four consecutive keys of one d column. Second read: keys key0 + 8...
  auto frag_offsets = [](int ln, int (&ko)[D / 16], int (&vo)[D / 32][2]) __attribute__((always_inline)) {
    const int r32 = ln & 31, h = ln >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ko[ks] = r32 * D + (((2 * ks + h) ^ swz<D>(r32)) << 3);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 4 * h + ((ln & 15) >> 2) + 8 * sec;          // row within a 16-row period
        const int ch = 4 * db + 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
        vo[db][sec] = r * D + ((ch ^ swz<D>(r)) << 3) + 4 * (ln & 1);
      }
  };
  // The offsets normally stay in registers for the whole loop. At d = 128 (where this
  // kernel runs the two-wave (64, 64) tile; the four-wave tiles there belong to the
  // pipelined kernel) the causal variant's loop otherwise spills (the accumulators,
  // Q^T and the previous tile's weights take most of 256 registers), so the offsets
  // are recomputed where they are used (one XOR and shift each) from a copy of the
  // lane index the compiler cannot hoist out of the loop (measured on the four-wave
  // (128, 64) tile: 449 -> 775 TFLOP/s); the other variants do not spill in their
  // main loop and only lose by the extra VALU work. The non-causal d = 128 variant
  // recomputes them in its masked tiles (the ragged last tile) only, where the mask's
  // registers made it spill (N = 1000, B = 8, H = 32: 683 -> 825).
  constexpr bool RECOMPUTE_OFFSETS = D == 128 && CAUSAL;
  constexpr bool RECOMPUTE_MASKED = RECOMPUTE_OFFSETS || (D == 128 && !CAUSAL && BN == 64);
  int koff_live[D / 16], voff_live[D / 32][2];
  frag_offsets(lane, koff_live, voff_live);
  auto fresh_offsets = [&](int (&ko)[D / 16], int (&vo)[D / 32][2]) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    frag_offsets(ln, ko, vo);
  };
  // Direct-to-LDS loads: load i of a tile fills LDS bytes [1024 i, 1024 i + 1024),
  // i.e. rows ROWS_PER_DMA*i.. of the tile; lane l fills tile row
  // ROWS_PER_DMA*i + 16 l / (2D), chunk position p = (16 l mod 2D) / 16, and so fetches
  // source chunk p ^ swz(row). This wave issues loads i = NW kk + wave, whose lane
  // offsets depend on i only through i mod PATS = ((NW kk) mod PATS + wave) mod PATS:
  // they are kept per value of (NW kk) mod PATS, a compile-time index (one or two
  // registers per tensor, not one per load). K and V may have different row
  // strides, so each has its own lane offsets.
  uint32_t dma_off_k[PATS], dma_off_v[PATS];
#pragma unroll
  for (int q = 0; q < PATS; ++q) {
    const int r_local = (16 * lane) / (2 * D);
    const int pch = ((16 * lane) % (2 * D)) / 16;
    const int r = ROWS_PER_DMA * ((q + wave) % PATS) + r_local;        // tile row mod 16
    const int col = (pch ^ swz<D>(r)) << 3;
    dma_off_k[q] = (uint32_t)((r_local * p.k_sr + col) * 2);
    dma_off_v[q] = (uint32_t)((r_local * p.v_sr + col) * 2);
  }
  // The 2-wave tile serves decoding (one to a few query rows per K/V head) and short
  // sequences, where every K/V byte is read about once: its loads are non-temporal
  // at d = 128 (measured on long-context decoding: 5.4 -> 5.7 TB/s at 32 key ranges,
  // 5.6 -> 6.4 at 64; neutral at d = 64, and 9-11% slower on the causal four-wave tiles,
  // whose K/V tiles are re-read from L2 by every row block).
  constexpr int LOAD_AUX = (NW == 2 && D == 128) ? 2 : 0;
  auto issue_tile_load = [&](const __amdgpu_buffer_rsrc_t& rsrc, const uint32_t (&lane_off)[PATS], int sr,
                             short* dst, int n0) {
#pragma unroll
    for (int kk = 0; kk < DMA_PER_WAVE; ++kk) {
      const int i = kk * NW + wave;
      buffer_load16_to_lds<LOAD_AUX>(rsrc, dst + 512 * i, lane_off[(kk * NW) % PATS],
                                     (uint32_t)((n0 + ROWS_PER_DMA * i) * sr * 2));
    }
  };

  // ---- Q^T as the B operand, kept in registers for the whole loop ----
  // qf[qb][ks] = Q[wq0 + 32 qb + l32][16 ks + 8 hi .. +7] (zeros past Nq).
  i16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[qb][ks] = buffer_load16(rq, (uint32_t)(((wq0 + 32 * qb + l32) * p.q_sr + ks * 16 + 8 * hi) * 2));

  f32x16 acc_o[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[qb][db][r] = 0.f;
  // Softmax state of each of this lane's queries: the exponent reference
  // ref = fl(c m_ref) (kept as the rounded product itself, so that
  // alpha = 2^(ref_old - ref_new) is exactly 1 for a row whose reference did not
  // move) and this lane's share of l.
  float ref[QB], nb[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { ref[qb] = -INFINITY; nb[qb] = 0.f; l_run[qb] = 0.f; }
  i16x8 pprev[QB][BN / 16];   // P of the previous tile as 16-bit B operands

  // Tile j holds keys kb + j BN ... Tiles [0, n_full) need no mask for any query of
  // this wave; the rest (the causal diagonal band and the ragged last tile) do.
  // Under a causal mask the workgroup's last query sees keys up to m0 + BM - 1 + off;
  // none may be visible. Every wave passes through all ntiles tiles (one barrier
  // each), the later waves of a causal workgroup with more of them unmasked.
  // Query indices of the workgroup's and the wave's rows: the rows themselves, or,
  // with query heads packed (qmod > 0), any of 0 .. qmod - 1.
  const bool packed = p.qmod > 0;
  const int wg_last_q = packed ? p.qmod - 1 : m0 + BM - 1;
  const int w_first_q = packed ? 0 : wq0;
  const int w_last_q = packed ? p.qmod - 1 : wq0 + 32 * QB - 1;
  const int n_end = CAUSAL ? min(ke, wg_last_q + 1 + off) : ke;
  const int ntiles = n_end > kb ? (n_end - kb + BN - 1) / BN : 0;
  const int full_end = CAUSAL ? min(ke, w_first_q + 1 + off) : ke;   // keys below it: valid for every query of the wave
  int n_full = full_end > kb ? (full_end - kb) / BN : 0;
  if (n_full > ntiles) n_full = ntiles;

  auto pv = [&](const short* vbuf, const int (&voff)[D / 32][2]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int tt = 0; tt < BN / 16; ++tt) {
        const short* src = vbuf + ((tt >> 1) * 32 + 16 * (tt & 1)) * D;
        const i16x4 a0 = ds_read_tr16(src + voff[db][0]);
        const i16x4 a1 = ds_read_tr16(src + voff[db][1]);
        const i16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc_o[qb][db] = mfma_32x32x16<BF16>(a, pprev[qb][tt], acc_o[qb][db]);
      }
    }
  };
  // Read-ahead of V (one query block per wave at d = 64): K(j) and V(j) arrive together
  // and share a stage index; each step reads its own V^T operands into registers at its
  // end, and the next step's MFMA section opens with P V from those registers while its
  // K reads are in flight, instead of waiting for LDS reads before its first MFMA.
  // Outputs are bit-identical. Measured: +1.9% to +2.1% on causal d = 64 workloads
  // (N = 1000 and 4096); with two query blocks per wave the operands do not fit beside
  // the rest (-0.5%, spills when read earlier), so that tile keeps the in-step reads.
  constexpr bool VPRE = D == 64 && QB == 1;
  i16x8 vfr[D / 32][BN / 16];   // V^T operands of the previous tile (VPRE)
  auto read_vfr = [&](const short* vbuf, const int (&voff)[D / 32][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int tt = 0; tt < BN / 16; ++tt) {
        const short* src = vbuf + ((tt >> 1) * 32 + 16 * (tt & 1)) * D;
        const i16x4 a0 = ds_read_tr16(src + voff[db][0]);
        const i16x4 a1 = ds_read_tr16(src + voff[db][1]);
        vfr[db][tt] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
  };
  auto pv_regs = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int tt = 0; tt < BN / 16; ++tt)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc_o[qb][db] = mfma_32x32x16<BF16>(vfr[db][tt], pprev[qb][tt], acc_o[qb][db]);
  };
  // P V outside a tile step (a causal tile in this wave's future, the last tile)
  auto pv_outside = [&](const short* vbuf) {
    if constexpr (RECOMPUTE_MASKED) {
      int ko_new[D / 16], vo_new[D / 32][2];
      fresh_offsets(ko_new, vo_new);
      pv(vbuf, vo_new);
    } else {
      pv(vbuf, voff_live);
    }
  };

  // One key tile: S = K(j) Q^T, then (if HAVE_PREV) the pending U += V(j-1)^T P(j-1)^T,
  // then the softmax of S into pprev.
  auto step = [&](int n0, const short* kbuf, const short* vprev, auto mask_tag, auto prev_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool HAVE_PREV = decltype(prev_tag)::value;
    // ---- S^T = K_tile Q^T: each K fragment feeds QB MFMAs ----
    constexpr bool PRIO_ALL = kRaisePvPriority && D == 64;
    constexpr bool FRESH = MASK ? RECOMPUTE_MASKED : RECOMPUTE_OFFSETS;
    int ko_new[D / 16], vo_new[D / 32][2];
    if constexpr (FRESH) fresh_offsets(ko_new, vo_new);
    const int(&koff)[D / 16] = FRESH ? ko_new : koff_live;
    const int(&voff)[D / 32][2] = FRESH ? vo_new : voff_live;
    f32x16 s[QB][BN / 32];
    if constexpr (PRIO_ALL) __builtin_amdgcn_s_setprio(2);
    if constexpr (VPRE && HAVE_PREV) pv_regs();
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const i16x8 a = *(const i16x8*)(kbuf + kb * 32 * D + koff[ks]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma_32x32x16<BF16>(a, qf[qb][ks], s[qb][kb]);
      }
    }
    // ---- the previous tile's P V: MFMA work that does not wait for this softmax ----
    if constexpr (HAVE_PREV && !VPRE) {
      if constexpr (kRaisePvPriority && !PRIO_ALL) __builtin_amdgcn_s_setprio(2);
      pv(vprev, voff);
    }
    if constexpr (kRaisePvPriority) __builtin_amdgcn_s_setprio(0);
    // s[qb][kb][r]: raw score of query wq0 + 32 qb + l32, key n0 + 32 kb + 8(r/4) + 4 hi + r%4.
    // A key is hidden when key >= Nk or (causal) key > query + off, i.e. when
    // key > lim = min(Nk - 1, query + off): one compare per score against the lane's
    // limit, measured from this lane's first key of the tile.
    if constexpr (MASK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        int query = wq0 + 32 * qb + l32;
        if (CAUSAL && packed) query %= p.qmod;
        const int lim = (CAUSAL ? min(Nk - 1, query + off) : Nk - 1) - (n0 + 4 * hi);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) s[qb][kb][r] = -INFINITY;
      }
    }

    // ---- online softmax ----
    // Weights against the current reference; their per-lane sum updates l and checks
    // the reference (the same rule as the eight-wave kernel's softmax: redo the tile
    // with references moved to the row maxima when a sum exceeds kSumMax, or on a
    // row's first tile).
    // Row sums: fp32 sums of the fp32 weights, or, for fp16 weights in unmasked tiles,
    // sums of the rounded weights formed mostly by packed fp16 adds (see kPackedSums).
    constexpr bool PACKED_SUM = kPackedSums && !BF16 && !MASK;
    auto weights = [&](float (&rs)[QB]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float part[2];
        e16x2 pairs[BN / 4];    // fp16 weights, two per register, for the fp16 row sum
#pragma unroll
        for (int tt = 0; tt < BN / 16; ++tt) {
          const int kb = tt >> 1, base = 8 * (tt & 1);
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kb][base + i], c, nb[qb]));
          e16x2 h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = __builtin_convertvector((f32x2){e[2 * i], e[2 * i + 1]}, e16x2);
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          pprev[qb][tt] = __builtin_bit_cast(i16x8, ((u32x4){__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                                              __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])}));
          if constexpr (!PACKED_SUM) {
            // the sums start from their first weights (not from 0 + weight: the same
            // value, one instruction less)
#pragma unroll
            for (int i = 0; i < 8; ++i) part[i & 1] = (tt == 0 && i < 2) ? e[i] : part[i & 1] + e[i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) pairs[4 * tt + i] = h[i];
          }
        }
        if constexpr (!PACKED_SUM) {
          rs[qb] = part[0] + part[1];
        } else {
          // two levels of packed fp16 adds (each half then sums four rounded weights),
          // the rest in fp32
          e16x2 q4[BN / 16];
#pragma unroll
          for (int i = 0; i < BN / 16; ++i) q4[i] = (pairs[4 * i] + pairs[4 * i + 1]) + (pairs[4 * i + 2] + pairs[4 * i + 3]);
          // then into one fp32 sum by mixed-precision FMAs (half * 1 + sum, one
          // v_fma_mix_f32 each, the first adding the two halves of a pair), which issue
          // as fast as an add, where a conversion costs half as much again
          float acc = __builtin_fmaf((float)q4[0].x, one, (float)q4[0].y);
#pragma unroll
          for (int i = 1; i < BN / 16; ++i) {
            acc = __builtin_fmaf((float)q4[i].x, one, acc);
            acc = __builtin_fmaf((float)q4[i].y, one, acc);
          }
          rs[qb] = acc;
        }
      }
    };
    float rs[QB];
    weights(rs);
    // After a full tile every row of the wave has a finite reference, so a full tile
    // that follows one only checks the sums.
    constexpr bool REF_SET = !MASK && HAVE_PREV;
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) redo |= !(rs[qb] <= kSumMax) || (!REF_SET && ref[qb] == -INFINITY);
    if (__builtin_amdgcn_ballot_w64(redo)) {   // wave-uniform: rare after the first tile
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        const float cand = max_halves(mx) * c;
        const float ref_new = cand > ref[qb] ? cand : ref[qb];
        // 1 if the reference did not move (also while it is still -inf: a row with no
        // visible key so far), 0 when it leaves -inf
        const float alpha = (ref_new == ref[qb]) ? 1.f : __builtin_amdgcn_exp2f(ref[qb] - ref_new);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_o[qb][db][r] *= alpha;    // after the pending P V landed
        ref[qb] = ref_new;
        nb[qb] = (ref_new == -INFINITY) ? 0.f : -ref_new;
      }
      weights(rs);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_run[qb] += rs[qb];
    if constexpr (VPRE) read_vfr(vprev, voff);   // V(j) is in LDS since this tile's barrier
  };

  // LDS stores by other waves' direct loads become visible after this wave's own
  // loads have landed (vmcnt) and everyone has passed the barrier.
  // With the read-ahead of V a wave's last V^T reads may still be in flight here; they
  // complete before the barrier, after which other waves' loads overwrite that stage.
  auto sync_tile = [&]() {
    if constexpr (VPRE)
      __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): also this wave's read-ahead of V
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads are in LDS
    __syncthreads();
  };

  // Tile j reads K(j) from stage j%2 and V(j-1) from stage (j-1)%2 while the direct
  // loads fill K(j+1) into stage (j+1)%2 and V(j) into stage j%2.
  // Without a causal mask the first iteration's loads (K(1), V(0)) start with K(0):
  // one memory round trip before the first tile instead of two. That matters where
  // every workgroup of the grid starts at once (n4096_d64_f16: +2.4%, N = 2048 and
  // 8192: +1.1% to +1.3%); under the causal mask, whose workgroups start staggered,
  // it measured 1-2% slower.
  constexpr bool EARLY = !CAUSAL;
  auto full_tile = [&](int j, short* k_rd, short* k_wr, short* v_rd, short* v_wr, auto prev_tag) {
    const int n0 = kb + j * BN;
    sync_tile();
    if constexpr (VPRE) {
      if ((!EARLY || j > 0) && j + 1 < ntiles) {
        issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + BN);
        issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0 + BN);
      }
    } else if (!EARLY || j > 0) {
      if (j + 1 < ntiles) issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + BN);
      issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0);
    }
    step(n0, k_rd, v_rd, std::false_type{}, prev_tag);
  };
  bool have_prev = false;   // pprev holds the weights of tile j-1 (wave-uniform)
  if (ntiles > 0) {
    issue_tile_load(rk, dma_off_k, p.k_sr, lds_k0, kb);
    if constexpr (VPRE) {
      // K(j) and V(j) share a stage index: tile j reads both from stage j%2
      issue_tile_load(rv, dma_off_v, p.v_sr, lds_v0, kb);
      if (EARLY && ntiles > 1) {
        issue_tile_load(rk, dma_off_k, p.k_sr, lds_k1, kb + BN);
        issue_tile_load(rv, dma_off_v, p.v_sr, lds_v1, kb + BN);
      }
    } else if (EARLY) {
      if (ntiles > 1) issue_tile_load(rk, dma_off_k, p.k_sr, lds_k1, kb + BN);
      issue_tile_load(rv, dma_off_v, p.v_sr, lds_v0, kb);
    }
  }
  int j = 0;
  // V stages: tile j reads V(j-1) from stage (j-1)%2, or with VPRE V(j) from stage j%2
  short* const v_even_rd = VPRE ? lds_v0 : lds_v1;
  short* const v_odd_rd = VPRE ? lds_v1 : lds_v0;
  if (n_full > 0) {
    full_tile(0, lds_k0, lds_k1, v_even_rd, v_odd_rd, std::false_type{});
    j = 1;
    for (; j + 1 < n_full; j += 2) {
      full_tile(j, lds_k1, lds_k0, v_odd_rd, v_even_rd, std::true_type{});
      full_tile(j + 1, lds_k0, lds_k1, v_even_rd, v_odd_rd, std::true_type{});
    }
    if (j < n_full) {
      full_tile(j, lds_k1, lds_k0, v_odd_rd, v_even_rd, std::true_type{});
      ++j;
    }
    have_prev = true;
  }
  for (; j < ntiles; ++j) {
    const int n0 = kb + j * BN;
    short* k_rd = (j & 1) ? lds_k1 : lds_k0;
    short* k_wr = (j & 1) ? lds_k0 : lds_k1;
    short* v_rd = (j & 1) ? v_odd_rd : v_even_rd;
    short* v_wr = (j & 1) ? v_even_rd : v_odd_rd;
    sync_tile();
    if constexpr (VPRE) {
      if ((!EARLY || j > 0) && j + 1 < ntiles) {
        issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + BN);
        issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0 + BN);
      }
    } else if (!EARLY || j > 0) {
      if (j + 1 < ntiles) issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + BN);
      issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0);
    }
    if (CAUSAL && n0 > w_last_q + off) {   // whole tile in this wave's future
      if (have_prev) {
        if constexpr (VPRE) pv_regs();
        else pv_outside(v_rd);
      }
      have_prev = false;
      continue;
    }
    if (have_prev) step(n0, k_rd, v_rd, std::true_type{}, std::true_type{});
    else step(n0, k_rd, v_rd, std::true_type{}, std::false_type{});
    have_prev = true;
  }
  if constexpr (VPRE) {
    if (have_prev) pv_regs();                   // the last tile's V^T operands are in registers
  } else {
    sync_tile();                                // V of the last tile is in LDS
    if (have_prev) pv_outside(((ntiles - 1) & 1) ? lds_v1 : lds_v0);
  }

  // ---- epilogue: O = U / l, LSE = ln2 (ref + log2 l) ----
  write_rows<D, BF16, QB>(p, sl, bh, wi.split, wq0, lane, acc_o, ref, l_run);
}

// Scheduling groups for one pipelined tile: NMF MFMAs, in chunks of QKT products
// S = K Q^T (one ds_read_b128 each) followed by PVT products U += V^T P^T (two
// transposing reads each). The LDS reads of MFMA i + PREF are issued after MFMA i,
// and VPM VALU instructions follow every MFMA.
template <int I, int NMF, int QKT, int PVT, int PREF, int VPM>
struct Interleave {
  static constexpr int reads(int i) { return (i % (QKT + PVT)) < QKT ? 1 : 2; }
  static constexpr int first() {
    int n = 0;
    for (int i = 0; i < PREF && i < NMF; ++i) n += reads(i);
    return n;
  }
  static __device__ __forceinline__ void emit() {
    if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, first(), 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);                              // VALU
    if constexpr (I + PREF < NMF) __builtin_amdgcn_sched_group_barrier(0x100, reads(I + PREF), 0);
    if constexpr (I + 1 < NMF) Interleave<I + 1, NMF, QKT, PVT, PREF, VPM>::emit();
  }
};

// ------------------------------------------------------------------------------------
// Software-pipelined kernel (four or eight waves)
// ------------------------------------------------------------------------------------
//
// On gfx950 one wave issues a VALU instruction only every ~6 cycles while the SIMD's
// VALU pipe accepts one every ~4 (v_exp_f32 holds it ~8.7 cycles), and a wave's
// MFMAs run on the matrix pipe while the same wave keeps issuing independent VALU
// instructions (measured with a probe of issue rates). So each wave interleaves, in
// one instruction stream, the softmax of tile j with the two products that do not
// depend on it: S(j+1) = K(j+1) Q^T and U += V(j-1)^T P(j-1)^T. Every tile of a wave
// is then one mixed stream of 16 (d = 64) or 32 (d = 128) MFMAs and ~113 VALU
// instructions, and the two waves of a SIMD fill both pipes without having to run
// in opposite phases.
//
// Iteration j (one barrier):
//   wait for this wave's loads, barrier     K(j+1), V(j-1) are in LDS stage (j+1)%2
//   start loads K(j+2), V(j) -> stage j%2   (their previous contents K(j), V(j-2) were
//                                            last read in iteration j-1)
//   softmax S(j) -> P(j)   interleaved with   S(j+1) = K(j+1) Q^T,  U += V(j-1)^T P(j-1)^T
// A reference move (rare) scales U after U += V(j-1)^T P(j-1)^T, which precedes it in
// program order, and before P(j) enters U one iteration later.
template <int D, bool BF16, bool CAUSAL, int NW, int BN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD))) void fa_fwd_pipe_kernel(Params p) {
#pragma clang fp contract(off)
  constexpr int BM = 32 * NW;
  constexpr int TILE = BN * D;
  constexpr int DMA_PER_TILE = TILE * 2 / 1024;
  constexpr int DMA_PER_WAVE = DMA_PER_TILE / NW;
  constexpr int ROWS_PER_DMA = 1024 / (2 * D);
  constexpr int PATS = 16 / ROWS_PER_DMA;
  constexpr int NKB = BN / 32, NKS = D / 16, NDB = D / 32, NTT = BN / 16;
  constexpr int NQK = NKB * NKS, NPV = NDB * NTT;      // MFMAs of each product per tile
  constexpr int QK_PER_TT = NQK / NTT, PV_PER_TT = NPV / NTT;
  static_assert(BN % 32 == 0 && (D == 64 || D == 128), "tile shape");
  static_assert(DMA_PER_TILE % NW == 0, "every wave issues the same number of loads");
  static_assert(NQK % NTT == 0 && NPV % NTT == 0, "products spread evenly over the softmax chunks");
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

  __shared__ __attribute__((aligned(1024))) short lds_k0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_k1[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v0[TILE];
  __shared__ __attribute__((aligned(1024))) short lds_v1[TILE];

  const WorkItem wi = work_item<CAUSAL, 8>(p);
  const int bh = wi.bh;
  const int Nk = p.Nk, off = p.causal_off;
  const int m0 = wi.mb * BM;
  const int kb = wi.split * p.split_keys;
  const int ke = min(Nk, kb + p.split_keys);
  const Slice sl = slice_of(p, bh);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(sl.q, p.q_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(sl.k, p.k_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(sl.v, p.v_bytes);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wq0 = m0 + wave * 32;
  const float c = p.c;

  // LDS fragment offsets, as in fa_fwd_kernel, in bytes
  auto frag_offsets = [](int ln, int (&ko)[NKS], int (&vo)[NDB][2]) __attribute__((always_inline)) {
    const int r32 = ln & 31, h = ln >> 5;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) ko[ks] = 2 * (r32 * D + (((2 * ks + h) ^ swz<D>(r32)) << 3));
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int r = 4 * h + ((ln & 15) >> 2) + 8 * sec;
        const int ch = 4 * db + 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
        vo[db][sec] = 2 * (r * D + ((ch ^ swz<D>(r)) << 3) + 4 * (ln & 1));
      }
  };
  int koff[NKS], voff[NDB][2];
  frag_offsets(lane, koff, voff);
  uint32_t dma_off_k[PATS], dma_off_v[PATS];
#pragma unroll
  for (int q = 0; q < PATS; ++q) {
    const int r_local = (16 * lane) / (2 * D);
    const int pch = ((16 * lane) % (2 * D)) / 16;
    const int r = ROWS_PER_DMA * ((q + wave) % PATS) + r_local;
    const int col = (pch ^ swz<D>(r)) << 3;
    dma_off_k[q] = (uint32_t)((r_local * p.k_sr + col) * 2);
    dma_off_v[q] = (uint32_t)((r_local * p.v_sr + col) * 2);
  }
  auto issue_tile_load = [&](const __amdgpu_buffer_rsrc_t& rsrc, const uint32_t (&lane_off)[PATS], int sr,
                             short* dst, int n0) {
#pragma unroll
    for (int kk = 0; kk < DMA_PER_WAVE; ++kk) {
      const int i = kk * NW + wave;
      buffer_load16_to_lds<0>(rsrc, dst + 512 * i, lane_off[(kk * NW) % PATS],
                              (uint32_t)((n0 + ROWS_PER_DMA * i) * sr * 2));
    }
  };

  i16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    qf[ks] = buffer_load16(rq, (uint32_t)(((wq0 + l32) * p.q_sr + ks * 16 + 8 * hi) * 2));
  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
  float ref = -INFINITY, nb = 0.f, l_run = 0.f;

  const bool packed = p.qmod > 0;
  const int wg_last_q = packed ? p.qmod - 1 : m0 + BM - 1;
  const int w_first_q = packed ? 0 : wq0;
  const int w_last_q = packed ? p.qmod - 1 : wq0 + 31;
  const int n_end = CAUSAL ? min(ke, wg_last_q + 1 + off) : ke;
  const int T = n_end > kb ? (n_end - kb + BN - 1) / BN : 0;          // tiles the workgroup streams
  int Tw = 0, n_full = 0;                                               // tiles this wave computes / needs no mask for
  if (wq0 < p.Nq) {
    const int w_end = CAUSAL ? min(ke, w_last_q + 1 + off) : ke;
    Tw = w_end > kb ? (w_end - kb + BN - 1) / BN : 0;
    if (Tw > T) Tw = T;
    const int full_end = CAUSAL ? min(ke, w_first_q + 1 + off) : ke;
    n_full = min(Tw, full_end > kb ? (full_end - kb) / BN : 0);
  }

  // ---- the pieces of one iteration ----
  // i-th MFMA of S = K Q^T (kb fastest, so that consecutive MFMAs are independent)
  auto qk_mfma = [&](f32x16 (&s)[NKB], const short* kbuf, int i, const int (&ko)[NKS]) __attribute__((always_inline)) {
    const int ks = i / NKB, kbk = i % NKB;
    const i16x8 a = *(const i16x8*)((const char*)(kbuf + kbk * 32 * D) + ko[ks]);
    s[kbk] = mfma_32x32x16<BF16>(a, qf[ks], ks == 0 ? f32x16{} : s[kbk]);
  };
  // i-th MFMA of U += V^T P^T (db fastest)
  auto pv_mfma = [&](const i16x8 (&pw)[NTT], const short* vbuf, int i, const int (&vo)[NDB][2]) __attribute__((always_inline)) {
    const int tt = i / NDB, db = i % NDB;
    const short* src = vbuf + ((tt >> 1) * 32 + 16 * (tt & 1)) * D;
    const i16x4 a0 = ds_read_tr16((const short*)((const char*)src + vo[db][0]));
    const i16x4 a1 = ds_read_tr16((const short*)((const char*)src + vo[db][1]));
    acc_o[db] = mfma_32x32x16<BF16>(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), pw[tt], acc_o[db]);
  };
  // weights of 16 keys (chunk tt) of s against the current reference, packed into pw[tt];
  // adds them to the two partial sums
  auto weights_chunk = [&](const f32x16 (&s)[NKB], i16x8 (&pw)[NTT], float (&part)[2], int tt) __attribute__((always_inline)) {
    const int kbk = tt >> 1, base = 8 * (tt & 1);
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kbk][base + i], c, nb));
    e16x2 h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_convertvector((f32x2){e[2 * i], e[2 * i + 1]}, e16x2);
    pw[tt] = __builtin_bit_cast(i16x8, ((u32x4){__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                                                 __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])}));
#pragma unroll
    for (int i = 0; i < 8; ++i) part[i & 1] = (tt == 0 && i < 2) ? e[i] : part[i & 1] + e[i];
  };
  // hidden scores to -inf: key > min(Nk - 1, query + off), one compare per score
  auto apply_mask = [&](f32x16 (&s)[NKB], int n0) __attribute__((always_inline)) {
    int query = wq0 + l32;
    if (CAUSAL && packed) query %= p.qmod;
    const int lim = (CAUSAL ? min(Nk - 1, query + off) : Nk - 1) - (n0 + 4 * hi);
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbk * 32 + 8 * (r >> 2) + (r & 3) > lim) s[kbk][r] = -INFINITY;
  };
  // After the weights of a tile: keep the reference while every lane's sum is at most
  // kSumMax; else (or on a row's first tile) move it to the row maximum, rescale l and
  // U (which already holds every earlier tile), and redo the weights.
  auto finish_softmax = [&](const f32x16 (&s)[NKB], i16x8 (&pw)[NTT], float rs) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(!(rs <= kSumMax) || ref == -INFINITY)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kbk][r]);
      const float cand = max_halves(mx) * c;
      const float ref_new = cand > ref ? cand : ref;
      const float alpha = (ref_new == ref) ? 1.f : __builtin_amdgcn_exp2f(ref - ref_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
      ref = ref_new;
      nb = (ref_new == -INFINITY) ? 0.f : -ref_new;
      float part[2];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) weights_chunk(s, pw, part, tt);
      rs = part[0] + part[1];
    }
    l_run += rs;
  };

  // Steady-state iteration: softmax of s_cur -> p_cur, interleaved with
  // s_next = K(j+1) Q^T and U += V(j-1)^T p_prev^T.
  auto body = [&](f32x16 (&s_cur)[NKB], f32x16 (&s_next)[NKB], i16x8 (&p_cur)[NTT], const i16x8 (&p_prev)[NTT],
                  const short* kbuf, const short* vbuf, int n0, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // The offsets pass through an empty asm once per tile, so the compiler cannot
    // hoist offset + stage address out of the loop: each stage's address then folds
    // into the reads' offset field, where hoisted sums would hold NKS + 2 * NDB
    // registers per stage (at d = 128 with 64-key tiles the loop would spill).
    // Not volatile, so that the asm does not split the scheduling region.
#pragma unroll
    for (int i = 0; i < NKS; ++i) asm("" : "+v"(koff[i]));
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm("" : "+v"(voff[i][h]));
    const int(&ko)[NKS] = koff;
    const int(&vo)[NDB][2] = voff;
    if constexpr (MASK) apply_mask(s_cur, n0);
    float part[2];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
      for (int m = 0; m < QK_PER_TT; ++m) qk_mfma(s_next, kbuf, tt * QK_PER_TT + m, ko);
#pragma unroll
      for (int m = 0; m < PV_PER_TT; ++m) pv_mfma(p_prev, vbuf, tt * PV_PER_TT + m, vo);
      weights_chunk(s_cur, p_cur, part, tt);
    }
    // Instruction order: the LDS reads run three MFMAs ahead of the MFMA that consumes
    // them; every MFMA is followed by an equal share of the softmax's VALU work (28
    // instructions per 16 keys: FMA, exp and add per weight, one pack per two).
    Interleave<0, NQK + NPV, QK_PER_TT, PV_PER_TT, 3, (28 * NTT) / (NQK + NPV)>::emit();
    // the packed weights are formed before the reference check (a redo rewrites them),
    // so that the packing joins the interleaved stream instead of trailing it
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) asm volatile("" ::"v"(p_cur[tt]));
    finish_softmax(s_cur, p_cur, part[0] + part[1]);
  };

  auto sync_tile = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
  };

  f32x16 s_a[NKB], s_b[NKB];
  i16x8 p_a[NTT], p_b[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) { p_a[tt] = (i16x8){}; p_b[tt] = (i16x8){}; }

  // ---- prologue: K(0) -> stage 0; S(0). V stage 1 is zeroed: the first main
  // iteration multiplies it by P(-1) = 0, and LDS may hold NaN patterns. ----
  if (T > 0) issue_tile_load(rk, dma_off_k, p.k_sr, lds_k0, kb);
#pragma unroll
  for (int i = tid * 8; i < TILE; i += NW * 64 * 8) *(i16x8*)(lds_v1 + i) = (i16x8){};
  sync_tile();
  if (T > 1) issue_tile_load(rk, dma_off_k, p.k_sr, lds_k1, kb + BN);
  if (Tw > 0) {
#pragma unroll
    for (int i = 0; i < NQK; ++i) qk_mfma(s_a, lds_k0, i, koff);
  }

  // ---- main loop: iterations j < n_main need no mask, and S(j+1) and P(j-1) are both
  // needed (P(-1) = 0 enters U harmlessly) ----
  const int n_main = min(n_full, Tw - 1);
  // iteration j reads K(j+1) and V(j-1) from stage (j+1)%2; loads K(j+2), V(j) into stage j%2
  auto main_iter = [&](int j, auto odd_tag) __attribute__((always_inline)) {
    constexpr bool ODD = decltype(odd_tag)::value;
    short* k_rd = ODD ? lds_k0 : lds_k1;
    short* v_rd = ODD ? lds_v0 : lds_v1;
    short* k_wr = ODD ? lds_k1 : lds_k0;
    short* v_wr = ODD ? lds_v1 : lds_v0;
    const int n0 = kb + j * BN;
    sync_tile();
    if (j + 2 < T) issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + 2 * BN);
    issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0);
    if constexpr (ODD) body(s_b, s_a, p_b, p_a, k_rd, v_rd, n0, std::false_type{});
    else body(s_a, s_b, p_a, p_b, k_rd, v_rd, n0, std::false_type{});
  };
  int j = 0;
  for (; j + 1 < n_main; j += 2) {
    main_iter(j, std::false_type{});
    main_iter(j + 1, std::true_type{});
  }
  // ---- tail: the rest of the tiles, one at a time, with the register sets swapped
  // to the even/odd naming by a copy when needed ----
  if (j < n_main) {
    // after an even iteration S(j+1) is in s_b and P(j) in p_a
    main_iter(j, std::false_type{});
    ++j;
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) s_a[kbk] = s_b[kbk];
  } else if (j > 0) {
    // after an odd iteration S(j+1) is in s_a and P(j) in p_b
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) p_a[tt] = p_b[tt];
  }
  bool have_prev = j > 0;    // p_a holds P(j-1)
  for (; j < T; ++j) {
    short* k_rd = (j & 1) ? lds_k0 : lds_k1;
    short* v_rd = (j & 1) ? lds_v0 : lds_v1;
    short* k_wr = (j & 1) ? lds_k1 : lds_k0;
    short* v_wr = (j & 1) ? lds_v1 : lds_v0;
    const int n0 = kb + j * BN;
    sync_tile();
    if (j + 2 < T) issue_tile_load(rk, dma_off_k, p.k_sr, k_wr, n0 + 2 * BN);
    issue_tile_load(rv, dma_off_v, p.v_sr, v_wr, n0);
    // S(j) is in s_a, P(j-1) in p_a
    if (j + 1 < Tw) {
#pragma unroll
      for (int i = 0; i < NQK; ++i) qk_mfma(s_b, k_rd, i, koff);
    }
    if (have_prev) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) pv_mfma(p_a, v_rd, i, voff);
    }
    have_prev = j < Tw;
    if (have_prev) {
      if (j >= n_full) apply_mask(s_a, n0);
      float part[2];
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) weights_chunk(s_a, p_a, part, tt);
      finish_softmax(s_a, p_a, part[0] + part[1]);
    }
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) s_a[kbk] = s_b[kbk];
  }
  sync_tile();                                   // V(T-1) is in LDS stage (T-1)%2
  if (have_prev) {
    const short* v_rd = ((T - 1) & 1) ? lds_v1 : lds_v0;
#pragma unroll
    for (int i = 0; i < NPV; ++i) pv_mfma(p_a, v_rd, i, voff);
  }
  float ref_a[1] = {ref}, l_a[1] = {l_run};
  f32x16 acc_w[1][NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_w[0][db] = acc_o[db];
  write_rows<D, BF16, 1>(p, sl, bh, wi.split, wq0, lane, acc_w, ref_a, l_a);
}

// ------------------------------------------------------------------------------------
// Split-KV merge
// ------------------------------------------------------------------------------------
//
// Each key range k of a query row left O_k (normalised by its own l_k) and LSE_k.
// Their combination is the attention over all keys: with LSE = ln sum_k e^(LSE_k),
// O = sum_k e^(LSE_k - LSE) O_k; a range with no visible key has LSE_k = -inf and
// weight 0, and a row with none at all gets O = 0, LSE = -inf. Memory-bound work:
// D / 2 lanes per row, two columns each. The lanes of a row share the LSE pass (each
// takes every (D/2)-th range, then a butterfly reduction) and leave the weights in
// LDS; the O pass issues its loads several ranges ahead.
constexpr int kMaxSplits = 256;

struct MergeParams {
  const float* po;
  const float* plse;
  short* o;
  float* lse;
  int rows;           // slices * Nq
  int Nq, Hq, splits;
  int o_sr;
  int64_t o_sb, o_sh;
};

template <int D, bool BF16, int G>
__global__ __launch_bounds__(256) void fa_merge_kernel(MergeParams m) {
#pragma clang fp contract(off)
  constexpr int LPR = D / 4;                 // lanes per row and group (4 columns each)
  constexpr int RPB = 256 / (LPR * G);       // rows per workgroup
  using f32x2 = float __attribute__((ext_vector_type(2)));
  using f32x4 = float __attribute__((ext_vector_type(4)));
  using e16x2 = typename std::conditional<BF16, __bf16 __attribute__((ext_vector_type(2))),
                                          _Float16 __attribute__((ext_vector_type(2)))>::type;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float wts[RPB][kMaxSplits];
  __shared__ f32x4 part[G > 1 ? RPB : 1][G][LPR];
  const int tid = (int)threadIdx.x;
  const int j = tid % LPR;                   // lane within the row's group
  const int grp = (tid / LPR) % G;           // group: ranges grp, grp + G, ...
  const int rl = tid / (LPR * G);            // row within the workgroup
  const int row = blockIdx.x * RPB + rl;
  const bool live = row < m.rows;
  const int64_t stride = m.rows;             // between the partials of consecutive ranges
  // every group forms the same weights; group 0 stores them
  float mx = -INFINITY;
  if (live)
    for (int k = j; k < m.splits; k += LPR) mx = fmaxf(mx, m.plse[k * stride + row]);
#pragma unroll
  for (int w = LPR / 2; w > 0; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w, LPR));
  float sum = 0.f;
  if (live && mx != -INFINITY)
    for (int k = j; k < m.splits; k += LPR) {
      const float e = __builtin_amdgcn_exp2f((m.plse[k * stride + row] - mx) * kLog2e);
      if (grp == 0) wts[rl][k] = e;
      sum += e;
    }
#pragma unroll
  for (int w = LPR / 2; w > 0; w >>= 1) sum += __shfl_xor(sum, w, LPR);
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (live && mx != -INFINITY) {             // sum >= 1: the maximal range contributes 1
    // the partials are read once: 16-byte non-temporal loads
    const f32x4* src = (const f32x4*)(m.po + (int64_t)row * D + 4 * j);
    const int64_t step = stride * D / 4;
    int k = grp;
    for (; k + 7 * G < m.splits; k += 8 * G) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(src + (k + u * G) * step);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += wts[rl][k + u * G] * x[u];
    }
    for (; k < m.splits; k += G) acc += wts[rl][k] * __builtin_nontemporal_load(src + k * step);
  }
  if constexpr (G > 1) {
    part[rl][grp][j] = acc;
    __syncthreads();
    if (grp != 0) return;
#pragma unroll
    for (int g = 1; g < G; ++g) acc += part[rl][g][j];
  }
  if (!live) return;
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    acc *= 1.f / sum;
    lse = mx + kLn2 * __builtin_amdgcn_logf(sum);
  }
  const int bh = row / m.Nq, i = row - bh * m.Nq;
  const int b = bh / m.Hq, h = bh - b * m.Hq;
  short* orow = m.o + b * m.o_sb + h * m.o_sh + (int64_t)i * m.o_sr + 4 * j;
  const e16x2 lo = __builtin_convertvector((f32x2){acc[0], acc[1]}, e16x2);
  const e16x2 hi2 = __builtin_convertvector((f32x2){acc[2], acc[3]}, e16x2);
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *(u32x2*)orow = (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi2)};
  if (j == 0) m.lse[row] = lse;
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------

template <int D, bool BF16>
hipError_t launch_merge(const MergeParams& m, hipStream_t stream) {
  // Few rows (decoding): eight lane groups per row share its ranges, so that the
  // grid has enough workgroups and each lane fewer dependent load rounds.
  constexpr int RPB1 = 256 / (D / 4), RPB8 = RPB1 / 8;
  if ((m.rows + RPB1 - 1) / RPB1 < 512)
    return launch_kernel(&fa_merge_kernel<D, BF16, 8>, (m.rows + RPB8 - 1) / RPB8, 256, stream, m);
  else
    return launch_kernel(&fa_merge_kernel<D, BF16, 1>, (m.rows + RPB1 - 1) / RPB1, 256, stream, m);
}

template <int D, bool BF16, bool CAUSAL, int NW, int BN, int QB = 1>
hipError_t launch_four_wave(const Params& p, hipStream_t stream) {
  if constexpr (CAUSAL || NW == 2)
    return fa_fwd_unit::launch_default_sched(p, D, BF16, CAUSAL, NW, BN, QB, stream);
  else
    return launch_kernel(&fa_fwd_kernel<D, BF16, CAUSAL, NW, QB, BN>, p.total_wgs, NW * 64, stream, p);
}

template <int D, bool BF16, bool CAUSAL, int NW, int BN>
hipError_t launch_pipelined(const Params& p, hipStream_t stream) {
  return launch_kernel(&fa_fwd_pipe_kernel<D, BF16, CAUSAL, NW, BN>, p.total_wgs, NW * 64, stream, p);
}

// The launch for a tile of kTiles (tile_ok has accepted it for this D).
template <int D, bool BF16, bool CAUSAL>
hipError_t launch_tile(const Params& p, int bm, int bn, hipStream_t stream) {
  if (bm == 64 && bn == 64) return launch_four_wave<D, BF16, CAUSAL, 2, 64>(p, stream);
  if (bm == 128 && bn == 64) {
    if constexpr (D == 64) return launch_four_wave<D, BF16, CAUSAL, 4, 64>(p, stream);
    else return launch_pipelined<D, BF16, CAUSAL, 4, 64>(p, stream);
  }
  if (bm == 128 && bn == 32) {
    if constexpr (D == 64) return launch_four_wave<D, BF16, CAUSAL, 4, 32>(p, stream);
    else return launch_pipelined<D, BF16, CAUSAL, 4, 32>(p, stream);
  }
  if (bm == 256 && bn == 32) {
    if constexpr (D == 64) return launch_four_wave<D, BF16, CAUSAL, 4, 32, 2>(p, stream);
    else return launch_pipelined<D, BF16, CAUSAL, 8, 32>(p, stream);
  }
  if (bm == 256 && bn == 64) return launch_pipelined<D, BF16, CAUSAL, 8, 64>(p, stream);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_d(const Params& p, bool bf16, bool causal, int bm, int bn, hipStream_t stream) {
  if (bf16) return causal ? launch_tile<D, true, true>(p, bm, bn, stream) : launch_tile<D, true, false>(p, bm, bn, stream);
  return causal ? launch_tile<D, false, true>(p, bm, bn, stream) : launch_tile<D, false, false>(p, bm, bn, stream);
}

#ifndef FA_FWD_DEFAULT_SCHED_UNIT

// Compiled tile shapes: block_m query rows per workgroup and block_n keys per K/V
// tile, and the head sizes each is built for. fa_fwd_kernel runs (64, 64) with two
// waves at both head sizes, (128, 64) and (128, 32) with four (32 query rows each)
// at d = 64, and (256, 32) at d = 64 with four waves of two 32-query blocks each
// (every K and V fragment read from LDS feeds both blocks); fa_fwd_pipe_kernel runs
// (128, 64) and (128, 32) at d = 128 with four waves and the eight-wave tiles
// (256, 32) at d = 128 and (256, 64) at both.
struct TileShape { int bm, bn; bool d64, d128; };
constexpr TileShape kTiles[] = {
    {64, 64, true, true}, {128, 64, true, true}, {128, 32, true, true}, {256, 32, true, true}, {256, 64, true, true}};

bool tile_ok(int64_t d, int bm, int bn) {
  if (d != 64 && d != 128) return false;
  for (const TileShape& t : kTiles)
    if (t.bm == bm && t.bn == bn) return d == 64 ? t.d64 : t.d128;
  return false;
}

// Row r of a slice with row stride sr is addressed as (r * sr + column) * 2 bytes in
// 32-bit arithmetic, for rows up to N + 512 (the padded last block).
bool rows_fit(int64_t N, int64_t sr) { return (N + 512) * sr < ((int64_t)1 << 30); }

// strides: {batch, head, row} in elements, non-negative multiples of 8 (16 bytes),
// row stride >= d; nullptr means contiguous [B, H, N, d].
fa_status read_strides(const int64_t* st, int64_t H, int64_t N, int64_t d, int64_t out[3]) {
  if (!st) {
    out[0] = H * N * d;
    out[1] = N * d;
    out[2] = d;
    return FA_OK;
  }
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0 || (st[i] & 7)) return FA_ERR_BAD_STRIDE;
    out[i] = st[i];
  }
  if (out[2] < d) return FA_ERR_BAD_STRIDE;
  return FA_OK;
}

// B H ceil(N / bm) >= need, without forming a product that could overflow.
bool grid_reaches(int64_t B, int64_t H, int64_t N, int64_t bm, int64_t need) {
  if (B <= 0 || H <= 0 || N <= 0) return false;
  const int64_t slices = (B >= need || H >= need) ? need : B * H;
  const int64_t per = N / bm + (N % bm != 0);      // row blocks per slice
  return per >= need || slices >= (need + per - 1) / per;
}

void default_tile(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int* bm, int* bn) {
  // Measured on MI355X (interleaved tile sweeps per workload family):
  //  - short sequences: the smallest tile, so that more workgroups exist;
  //  - d = 64: the four-wave kernel. Without a mask, two 32-query blocks per wave
  //    (256 rows, 32-key tiles: the K and V fragments read from LDS serve both) where
  //    that grid still gives every CU two workgroups (+2.4% to +3.5% at N = 2048 to
  //    16384; with one per CU, -16%); otherwise one block per wave (causal row blocks
  //    of uneven length balance better with small blocks): 64-key tiles for
  //    non-causal sequences (+3.6% to +8% over 32-key ones at N = 1024 to 4096 with 8
  //    or 16 heads); under a causal mask 64-key tiles (two workgroups per CU) while the
  //    128-row grid is at most one round of 512 workgroups (+7.6% to +11% at N = 512 to
  //    2048), or 1.5 rounds from N = 2048 (+11% at N = 3072), and 32-key tiles (three
  //    workgroups per CU) beyond (64 keys: -9.4% to +0.2% at 1024 to 4096 workgroups,
  //    except +4.5% at N = 8192 with 1024); the pipelined kernel measured 3% slower
  //    at N = 4096 (the softmax's VALU work, not the overlap, sets the pace there);
  //  - d = 128: the pipelined kernel. Eight waves for long sequences (one workgroup
  //    of 256 rows per CU streams each K/V tile once for twice the rows: +1.7% to
  //    +2.3% at N = 16384 without a mask, +1.5% to +3.2% at N = 4096 to 16384 with
  //    one), provided the 256-row grid covers the 256 CUs (without a mask) or twice
  //    that (with one, whose row blocks differ in length): below that the 128-row tile
  //    was 19% to 35% faster (N = 4096 and 8192, 8 heads). 64-key tiles from N = 4096
  //    (+2.3% to +5% over 32-key ones with 256 rows, +3.4% to +8.3% with 128), for
  //    shorter sequences without a mask (within 1% of the 32-key and four-wave tiles)
  //    and for shorter causal ones whose 128-row grid is one round of two workgroups
  //    per CU (+2.3% to +15% at N = 1024 to 3072); 32-key tiles for causal ones with
  //    more workgroups than that (from -2.5% to +2% for 64 keys) and up to N = 256.
  if (N <= 128) {
    *bm = 64;
    *bn = 64;
  } else if (d == 128) {
    const bool eight = N >= 4096 && grid_reaches(B, H, N, 256, causal ? 512 : 256);
    *bm = eight ? 256 : 128;
    const bool causal_rounds = causal && N < 4096 && grid_reaches(B, H, N, 128, 513);
    *bn = (N > 256 && !causal_rounds) ? 64 : 32;
  } else {
    const bool two_blocks = !causal && N > 256 && grid_reaches(B, H, N, 256, 512);
    *bm = two_blocks ? 256 : 128;
    if (two_blocks || N <= 256) {
      *bn = 32;
    } else if (!causal) {
      *bn = 64;
    } else {
      const bool one_round = !grid_reaches(B, H, N, 128, 513);
      const bool rounds_and_half = N >= 2048 && !grid_reaches(B, H, N, 128, 769);
      *bn = one_round || rounds_and_half ? 64 : 32;
    }
  }
}


// Resident workgroups per CU, from each tile's registers (a SIMD holds 512 per
// lane): the four-wave tiles of both kernels run one wave per SIMD per workgroup,
// two workgroups per CU at 169..256 registers and three for the 32-key tiles at
// d = 64 (at most 168);
// the 2-wave (64, 64) tile fits two waves per SIMD at d = 64 (4 per CU) but needs
// more than 256 registers at d = 128 (2 per CU); the four-wave (256, 32) tile at
// d = 64 (two query blocks per wave, 255 registers) two per CU; an eight-wave
// workgroup fills a CU.
int wgs_per_cu(int bm, int bn, int64_t d) {
  if (bm == 64) return d == 64 ? 4 : 2;
  if (bm == 128) return (d == 64 && bn == 32) ? 3 : 2;
  if (bm == 256 && bn == 32 && d == 64) return 2;
  return 1;
}

// Key ranges per query block for split-KV. Measured on MI355X: a split pays when the
// query blocks leave resident workgroup slots empty, and pays best when every slot is
// filled once (a second round of workgroups costs more than the shorter ranges save)
// with ranges of at least 8 key tiles, below which the per-workgroup prologue and
// the merge dominate. Decoding-like shapes (a single, mostly empty query block per
// slice) stream K and V at the memory's pace and do best with two workgroups per CU
// (measured with non-temporal loads: 6.4 against 5.7 TB/s with one per CU at d = 128,
// 5.6 against 5.0 at d = 64, 32 query heads over 8 K/V heads, 128K keys).
// Grouped query heads with fewer rows than this per head are packed into one slice
// per K/V head (decoding, a few draft tokens): one K/V stream serves the whole group.
constexpr int64_t kPackRows = 64;
bool packs_heads(int64_t Nq) { return Nq >= 1 && Nq < kPackRows; }

int split_heuristic(int64_t B, int64_t Hq, int64_t Nq, int64_t Nk, int64_t d, int bm, int bn) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nk <= 0) return 1;
  const int64_t base = B * Hq * ((Nq + bm - 1) / bm);
  const int64_t slots = 256 * (int64_t)(2 * Nq <= bm ? 2 : wgs_per_cu(bm, bn, d));
  if (base >= slots) return 1;
  const int64_t tiles = (Nk + bn - 1) / bn;
  int64_t sp = slots / base;
  if (sp > tiles / 8) sp = tiles / 8;
  if (sp > kMaxSplits) sp = kMaxSplits;
  return sp < 1 ? 1 : (int)sp;
}

// ------------------------------------------------------------------------------------
// Built-in scratch for the allocation-free split-KV entry point
// ------------------------------------------------------------------------------------
//
// One array per GPU, as large as the biggest split-KV partial set this entry point
// accepts; it lives until the process ends. Host code never passes the array's name
// to a kernel (on the host it only stands for the symbol): its device address is
// looked up once per device, with that device current, and kept here.
constexpr size_t kScratchBytes = FA_SPLIT_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, or null on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// Everything fa_fwd, fa_fwd_ex and fa_fwd_split share. num_splits = 1: one workgroup
// per query block, written straight to o and lse; otherwise partials in workspace
// and a merge launch.
fa_status run(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
              int64_t Hk, int64_t Nq, int64_t Nk, int64_t d, const int64_t* qs_in, const int64_t* ks_in,
              const int64_t* vs_in, const int64_t* os_in, float scale, int causal, fa_dtype dtype,
              hipStream_t stream, int bm, int bn, int num_splits = 1, void* workspace = nullptr,
              size_t workspace_bytes = 0, bool use_scratch = false) {
  if (B < 0 || Hq < 0 || Hk < 0 || Nq < 0 || Nk < 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEADDIM;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_BAD_DTYPE;
  const bool auto_tile = bm == 0 && bn == 0;
  if (!auto_tile && !tile_ok(d, bm, bn)) return FA_ERR_UNSUPPORTED_TILE;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_BAD_SPLITS;
  if (B == 0 || Hq == 0 || Nq == 0) return FA_OK;
  if (Hk == 0 || Hq % Hk != 0) return FA_ERR_BAD_SHAPE;
  if (!q || !o || !lse) return FA_ERR_NULL_PTR;
  if (Nk > 0 && (!k || !v)) return FA_ERR_NULL_PTR;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15) return FA_ERR_MISALIGNED;
  if ((uintptr_t)lse & 3) return FA_ERR_MISALIGNED;
  int64_t qs[3], ks[3], vs[3], os[3];
  fa_status st;
  if ((st = read_strides(qs_in, Hq, Nq, d, qs)) != FA_OK) return st;
  if ((st = read_strides(ks_in, Hk, Nk, d, ks)) != FA_OK) return st;
  if ((st = read_strides(vs_in, Hk, Nk, d, vs)) != FA_OK) return st;
  if ((st = read_strides(os_in, Hq, Nq, d, os)) != FA_OK) return st;
  int64_t group = Hq / Hk;
  // Decoding with grouped K/V heads (fewer than kPackRows query rows per head): the
  // query heads that share a K/V head become the rows of one slice, so that one
  // workgroup streams each K/V tile once for all of them. With one row per head the
  // rows are one head stride apart (and the bottom-right causal mask hides no key);
  // with Nq rows per head q and o must be head-contiguous (head stride = Nq row
  // strides), so that row g Nq + i of the slice is query i of head g, and the kernel
  // takes the query index for the causal mask as row mod Nq. The lse rows
  // [B, Hq, Nq] are [B, Hk, group Nq] either way.
  int64_t qmod = 0;
  if (group > 1 && packs_heads(Nq) && (Nq == 1 || (qs[1] == Nq * qs[2] && os[1] == Nq * os[2]))) {
    if (Nq == 1) {
      qs[2] = qs[1];        // row r of the packed slice: query head r of the group
      os[2] = os[1];
      causal = 0;
    } else {
      qmod = Nq;
    }
    qs[1] *= group;         // next slice: the next group of query heads
    os[1] *= group;
    Nq *= group;
    Hq = Hk;
    group = 1;
  }
  if (auto_tile) default_tile(B, Hq, Nq, d, causal, &bm, &bn);
  if (!rows_fit(Nq, qs[2]) || !rows_fit(Nq, os[2]) || !rows_fit(Nk, ks[2]) || !rows_fit(Nk, vs[2]))
    return FA_ERR_TOO_LARGE;
  if (B >= ((int64_t)1 << 31) || Hq >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  const int64_t slices = B * Hq;
  if (slices >= ((int64_t)1 << 31) / Nq + 1) return FA_ERR_TOO_LARGE;   // rows = slices * Nq < 2^31
  const int64_t mblocks = (Nq + bm - 1) / bm;
  // key ranges: a whole number of tiles each, none empty
  const int64_t tiles = (Nk + bn - 1) / bn;
  int64_t splits = num_splits < tiles ? num_splits : (tiles > 0 ? tiles : 1);
  int64_t split_keys = ((tiles + splits - 1) / splits) * bn;
  if (Nk > 0) splits = (Nk + split_keys - 1) / split_keys;
  if (splits == 1) split_keys = tiles * bn;
  const int64_t total = slices * mblocks * splits;
  if (total >= ((int64_t)1 << 31)) return FA_ERR_TOO_LARGE;
  float* po = nullptr;
  float* plse = nullptr;
  if (splits > 1) {
    const int64_t rows = slices * Nq;
    const uint64_t need = (uint64_t)splits * rows * (d + 1) * 4;
    if (use_scratch) {
      // the built-in scratch: looked up only once every argument has passed
      if (need > kScratchBytes) return FA_ERR_SCRATCH_LIMIT;
      workspace = device_scratch();
      if (!workspace) return FA_ERR_HIP;
      workspace_bytes = kScratchBytes;
    }
    if (!workspace || ((uintptr_t)workspace & 15) || workspace_bytes < need) return FA_ERR_WORKSPACE;
    po = (float*)workspace;
    plse = po + splits * rows * d;
  }
  Params p;
  p.q = (const short*)q;
  p.k = (const short*)k;
  p.v = (const short*)v;
  p.o = (short*)o;
  p.lse = lse;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.Hq = (int)Hq;
  p.group = (int)group;
  p.causal_off = (int)(Nk - (qmod > 0 ? qmod : Nq));   // bottom-right alignment; 0 (top-left) when Nq = Nk
  p.qmod = (int)qmod;
  p.q_sb = qs[0]; p.q_sh = qs[1]; p.q_sr = (int)qs[2];
  p.k_sb = ks[0]; p.k_sh = ks[1]; p.k_sr = (int)ks[2];
  p.v_sb = vs[0]; p.v_sh = vs[1]; p.v_sr = (int)vs[2];
  p.o_sb = os[0]; p.o_sh = os[1]; p.o_sr = (int)os[2];
  p.q_bytes = (uint32_t)((Nq - 1) * qs[2] + d) * 2;
  p.k_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * ks[2] + d) * 2 : 0;
  p.v_bytes = Nk > 0 ? (uint32_t)((Nk - 1) * vs[2] + d) * 2 : 0;
  p.num_m_blocks = (int)mblocks;
  p.num_splits = (int)splits;
  p.split_keys = (int)split_keys;
  p.slices = (int)slices;
  p.total_wgs = (int)total;
  p.c = (float)((double)scale * 1.4426950408889634);  // s * log2(e), rounded once
  p.po = po;
  p.plse = plse;
  const hipStream_t s = stream;
  const bool bf16 = dtype == FA_BF16;
  hipError_t e = (d == 64) ? launch_d<64>(p, bf16, causal != 0, bm, bn, s)
                           : launch_d<128>(p, bf16, causal != 0, bm, bn, s);
  if (e == hipSuccess && splits > 1) {
    MergeParams m;
    m.po = po;
    m.plse = plse;
    m.o = (short*)o;
    m.lse = lse;
    m.rows = (int)(slices * Nq);
    m.Nq = (int)Nq;
    m.Hq = (int)Hq;
    m.splits = (int)splits;
    m.o_sr = (int)os[2];
    m.o_sb = os[0];
    m.o_sh = os[1];
    if (d == 64) e = bf16 ? launch_merge<64, true>(m, s) : launch_merge<64, false>(m, s);
    else e = bf16 ? launch_merge<128, true>(m, s) : launch_merge<128, false>(m, s);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                 int64_t H, int64_t N, int64_t d, float scale, int causal, fa_dtype dtype,
                 hipStream_t stream) {
  int bm, bn;
  default_tile(B, H, N, d, causal, &bm, &bn);
  return run(q, k, v, o, lse, B, H, H, N, N, d, nullptr, nullptr, nullptr, nullptr, scale, causal, dtype,
             stream, bm, bn);
}

fa_status fa_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                       int64_t H, int64_t N, int64_t d, float scale, int causal, fa_dtype dtype,
                       hipStream_t stream, int block_m, int block_n) {
  if (block_m == 0 && block_n == 0) block_m = -1;   // no automatic choice here: (0, 0) is not a tile
  return run(q, k, v, o, lse, B, H, H, N, N, d, nullptr, nullptr, nullptr, nullptr, scale, causal, dtype,
             stream, block_m, block_n);
}

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                    int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d, const int64_t* q_strides,
                    const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
                    float scale, int causal, fa_dtype dtype, hipStream_t stream, int block_m, int block_n) {
  return run(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides, scale,
             causal, dtype, stream, block_m, block_n);
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                       int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d, const int64_t* q_strides,
                       const int64_t* k_strides, const int64_t* v_strides, const int64_t* o_strides,
                       float scale, int causal, fa_dtype dtype, hipStream_t stream, int block_m, int block_n,
                       int num_splits, void* workspace, size_t workspace_bytes) {
  return run(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides, scale,
             causal, dtype, stream, block_m, block_n, num_splits, workspace, workspace_bytes);
}

fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                               int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d,
                               const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                               const int64_t* o_strides, float scale, int causal, fa_dtype dtype, hipStream_t stream,
                               int block_m, int block_n, int num_splits) {
  // the partials of num_splits ranges must fit the built-in scratch: the same bound as
  // the workspace size of the caller-workspace form, checked before any HIP call
  if (num_splits > 1 && B > 0 && Hq > 0 && Nq > 0 && (d == 64 || d == 128) && num_splits <= kMaxSplits) {
    const double need = (double)num_splits * (double)B * (double)Hq * (double)Nq * (double)(d + 1) * 4.0;
    if (need > (double)kScratchBytes) return FA_ERR_SCRATCH_LIMIT;
  }
  return run(q, k, v, o, lse, B, Hq, Hk, Nq, Nk, d, q_strides, k_strides, v_strides, o_strides, scale, causal,
             dtype, stream, block_m, block_n, num_splits, nullptr, 0, true);
}

size_t fa_split_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d, int num_splits) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || (d != 64 && d != 128) || num_splits < 1 || num_splits > kMaxSplits) return 0;
  if (num_splits == 1) return 0;
  return (size_t)num_splits * (size_t)(B * Hq * Nq) * (size_t)(d + 1) * 4;
}

int fa_split_default(int64_t B, int64_t Hq, int64_t Hk, int64_t Nq, int64_t Nk, int64_t d, int causal,
                     int block_m, int block_n) {
  if (B <= 0 || Hq <= 0 || Hk <= 0 || Hq % Hk || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 1;
  if (Hq > Hk && packs_heads(Nq)) {   // grouped heads with few rows: the group forms one slice
    if (Nq == 1) causal = 0;            // (assuming head-contiguous q and o when Nq > 1)
    Nq *= Hq / Hk;
    Hq = Hk;
  }
  if (block_m == 0 && block_n == 0) default_tile(B, Hq, Nq, d, causal, &block_m, &block_n);
  if (!tile_ok(d, block_m, block_n)) return 1;
  return split_heuristic(B, Hq, Nq, Nk, d, block_m, block_n);
}

int fa_tile_supported(int64_t d, int block_m, int block_n) { return tile_ok(d, block_m, block_n) ? 1 : 0; }

fa_status fa_default_tile(int64_t B, int64_t H, int64_t N, int64_t d, int causal, int* block_m,
                          int* block_n) {
  if (!block_m || !block_n) return FA_ERR_NULL_PTR;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_HEADDIM;
  default_tile(B, H, N, d, causal, block_m, block_n);
  return FA_OK;
}

const char* fa_status_str(fa_status status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "null pointer";
    case FA_ERR_BAD_SHAPE: return "negative size, or Hq not a positive multiple of Hk";
    case FA_ERR_UNSUPPORTED_HEADDIM: return "head dimension must be 64 or 128";
    case FA_ERR_BAD_SCALE: return "scale must be finite and > 0";
    case FA_ERR_BAD_DTYPE: return "dtype must be FA_F16 or FA_BF16";
    case FA_ERR_MISALIGNED: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_TOO_LARGE: return "problem too large ((N + 512) * row stride >= 2^30 or grid >= 2^31)";
    case FA_ERR_UNSUPPORTED_TILE: return "tile shape not compiled";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_BAD_STRIDE: return "strides must be non-negative multiples of 8 elements, row stride >= d";
    case FA_ERR_BAD_SPLITS: return "num_splits must be between 1 and 256";
    case FA_ERR_WORKSPACE: return "split-KV workspace missing, not 16-byte aligned or smaller than fa_split_workspace_bytes";
    case FA_ERR_SCRATCH_LIMIT: return "split-KV partials exceed the built-in scratch (FA_SPLIT_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"

#else  // FA_FWD_DEFAULT_SCHED_UNIT

template <int D, bool BF16, bool CAUSAL, int NW, int BN, int QB>
hipError_t launch_here(const Params& p, hipStream_t stream) {
  return launch_kernel(&fa_fwd_kernel<D, BF16, CAUSAL, NW, QB, BN>, p.total_wgs, NW * 64, stream, p);
}

// The tiles launch_four_wave sends here: (64, 64) with two waves for either mask and
// head size, and the d = 64 four-wave tiles under a causal mask.
template <int D, bool BF16, bool CAUSAL>
hipError_t launch_masked_or_two_wave(const Params& p, int nw, int bn, int qb, hipStream_t stream) {
  if (nw == 2 && bn == 64 && qb == 1) return launch_here<D, BF16, CAUSAL, 2, 64, 1>(p, stream);
  if constexpr (D == 64 && CAUSAL) {
    if (nw == 4 && bn == 64 && qb == 1) return launch_here<64, BF16, true, 4, 64, 1>(p, stream);
    if (nw == 4 && bn == 32 && qb == 1) return launch_here<64, BF16, true, 4, 32, 1>(p, stream);
    if (nw == 4 && bn == 32 && qb == 2) return launch_here<64, BF16, true, 4, 32, 2>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t fa_fwd_unit::launch_default_sched(const Params& p, int d, bool bf16, bool causal, int nw, int bn, int qb,
                                             hipStream_t stream) {
  if (d == 64) {
    if (bf16) return causal ? launch_masked_or_two_wave<64, true, true>(p, nw, bn, qb, stream)
                            : launch_masked_or_two_wave<64, true, false>(p, nw, bn, qb, stream);
    return causal ? launch_masked_or_two_wave<64, false, true>(p, nw, bn, qb, stream)
                  : launch_masked_or_two_wave<64, false, false>(p, nw, bn, qb, stream);
  }
  if (bf16) return causal ? launch_masked_or_two_wave<128, true, true>(p, nw, bn, qb, stream)
                          : launch_masked_or_two_wave<128, true, false>(p, nw, bn, qb, stream);
  return causal ? launch_masked_or_two_wave<128, false, true>(p, nw, bn, qb, stream)
                : launch_masked_or_two_wave<128, false, false>(p, nw, bn, qb, stream);
}

#endif  // FA_FWD_DEFAULT_SCHED_UNIT
