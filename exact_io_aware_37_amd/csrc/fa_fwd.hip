// Exact tiled attention forward for gfx950 (MI355X): kernels and C ABI.
//
// One workgroup owns BR consecutive query rows of one (batch, query head).
// It keeps, per row, an exponent reference m, a running exponential sum l and
// an fp32 output accumulator in registers, streams the key/value sequence in
// tiles through LDS, and after the last tile divides by l once and writes O
// and lse.  This is the recurrence of the course page "FlashAttention:
// IO-aware attention kernel" (section 3.2: new max, rescale the old sum and
// accumulator by exp(m_old - m_new), add the tile's exponentials) inside the
// query-tile-outer / key-tile-inner loop of its sections 2 and 3.3.  The
// omica exam notes (section 2.3, block merge rule) state the same update for
// whole tiles.  Scores and probabilities exist only in registers; nothing of
// size N_q x N_kv touches memory.
//
// Matrix-core mapping (wave64, 32 query rows per wave):
//   S^T = K Q^T   v_mfma_f32_32x32x16_{bf16,f16}: A = K rows from LDS, B = Q^T
//                 held in registers for the whole loop.  The accumulator puts
//                 one query per lane (lane % 32) and 16 keys per lane in
//                 registers, so the row max and row sum are in-lane except
//                 for one exchange between the two half-waves.
//   O^T += V^T P^T  same instruction: B = P^T straight from the S^T
//                 accumulator (rounded to the input type), A = V^T read from
//                 row-major V in LDS by ds_read_b64_tr_b16, which hands each
//                 lane 4 keys of one head-dimension column; the key order of
//                 the accumulator is matched by the choice of rows each lane
//                 reads.  The output accumulator also has one query per lane,
//                 so the rescale factor and the final 1/l are lane-local.
// The fp32 variant uses v_mfma_f32_32x32x2_f32 with a simpler skeleton.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fa.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// Launch-independent arguments shared by every kernel variant.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nkv;
  int group;      // Hq / Hkv: query heads per key/value head
  int n_qtiles;   // ceil(Nq / BR)
  int n_heads;    // B * Hq
  float sl2;      // |scale| * log2(e), or 1 when scale == 0
  int qmode;      // 0: Q as given, 1: negated (scale < 0), 2: zeroed (scale == 0)
  float oscale;   // factor applied to O at the end (FP8 path: V's dequantisation factor)
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// Work item of this workgroup.  Non-causal grids are remapped so that the
// hardware's round-robin dispatch over the 8 XCDs (block i runs on XCD i % 8)
// hands each XCD a contiguous range of (head, query tile) items: the tiles
// of one head, which read the same K/V, then share that XCD's L2.  Causal
// grids keep the dispatch order and list the longest tiles (the last query
// tiles) first, heads fastest, so that the triangular work drains evenly.
__device__ __forceinline__ void map_block(const Params& p, bool causal, int& b, int& hq,
                                          int& qt) {
  const int bid = blockIdx.x;
  const int nb = gridDim.x;
  int hl;
  if (!causal) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int per = nb >> 3, rem = nb & 7;
    const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
    hl = logical / p.n_qtiles;
    qt = logical - hl * p.n_qtiles;
  } else {
    const int r = bid / p.n_heads;
    hl = bid - r * p.n_heads;
    qt = p.n_qtiles - 1 - r;
  }
  b = hl / p.Hq;
  hq = hl - b * p.Hq;
}

// Block index renumbered so that each XCD (dispatch is round-robin: block i
// runs on XCD i % 8) receives one contiguous range of logical indices.
__device__ __forceinline__ int xcd_local(int bid, int nb) {
  const int xcd = bid & 7, slot = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// ----------------------------------------------- 16-bit (bf16 / f16) path
//
// Helpers and layouts shared by the 16-bit kernels: the forward (attn_fwd_w64,
// 64 query rows per wave, at d = 64 and 128), split-KV, paged and backward.
// K/V tiles move global -> LDS by buffer DMA (buffer_load ... lds, 16 B per
// lane, no VGPR staging; rows past N_kv come back as zeros).  K is stored
// row-major with an XOR swizzle of its 16-byte chunks (conflict-free 16-byte
// operand reads); V is stored row-major too, with its own swizzle, and read
// transposed by ds_read_b64_tr_b16, which hands each lane four keys of one
// head-dimension column: the V^T operand of the P*V product without any
// transpose pass.
//
// The exponent reference is lazy: it moves to the new running max only when
// that max exceeds it by more than 2^8 (then O and the sum are rescaled by
// exp2(m_old - m_new)).  Otherwise probabilities are taken against the older,
// smaller reference and stay below 2^8.  O / l and lse = ref + log2(l) are
// the same whatever reference is used, so the result stays exact; only the
// rescale work is skipped.  The kernels of this file use 2^8 (kLazy; the FP8
// path needs it: E4M3's largest value is 448); the generated 64-row forward
// body uses 2^15, as much as f16 probabilities allow (largest value 65504).

typedef __attribute__((address_space(3))) unsigned char lds_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr float kLazy = 8.0f;   // log2 of the largest probability the lazy reference allows

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // Raw buffer (stride 0): loads past `bytes` return zero, stores past it are dropped.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all its LDS operations completed (s_waitcnt vmcnt(N) lgkmcnt(0)).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// Combine the two half-waves' values of a lane pair (l, l ^ 32) with
// v_permlane32_swap; both lanes of a pair get the same, bitwise-identical
// result (max and + are commutative).
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
struct Mma16;

template <>
struct Mma16<__bf16> {
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  // acc + lo + hi of a packed pair, accumulated in fp32.
  __device__ static __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
  }
  // acc + a.lo * b.lo + a.hi * b.hi of two packed pairs, in fp32.
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
  }
};

template <>
struct Mma16<_Float16> {
  __device__ static __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair),
                                  __builtin_bit_cast(f16x2, 0x3c003c00u), acc, false);
  }
  __device__ static __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc,
                                  false);
  }
};

// XOR swizzles of the 16-byte chunk index within a row (period 16 rows).
// K: 16 consecutive rows read the same logical chunk -> 16 distinct chunks.
// V: a transposed read touches 4 consecutive rows x 4 chunks -> 16 distinct.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}
// Tiles read both ways (row reads for one product, ds_read_b64_tr_b16 for the
// other: Q, dO and K in the backward): the chunk index XOR
// 4 * (row % 4) + (row / 4) % 4 at d = 128, 4 * ((row / 2) % 2) + (row / 4) % 4
// at d = 64.  16 consecutive rows still see 16 distinct chunks (8 per row
// parity at d = 64), and the 4 rows of a transposed read see 4 distinct
// groups of 4 chunks, so neither read has a bank conflict (64 banks of 4 bytes).
template <int D>
__device__ __forceinline__ int swz_kt(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// ------------------------------- 64 rows per wave (bf16 / f16, d = 64 and 128)
//
// The forward of the 16-bit inputs: each wave owns 64 query rows, one wave
// per SIMD (4 waves, 256 rows per workgroup), and every K and V fragment read
// from LDS feeds two matrix instructions (one per 32-row half).  O and Q
// live in accumulation registers, scores and probabilities in vector
// registers; that split, the register
// assignment and the instruction schedule are written out by
// gen_fwd_w64.py, whose header describes them, into fa_fwd_w64.inc, and the
// whole per-workgroup computation (Q load, the K/V DMA ring of 4 stages
// issued 3 tiles ahead, one barrier per tile, masking of ragged and
// causal-diagonal tiles, the lazy exponent reference, the epilogue with
// O staged through LDS for whole-row stores) runs in one inline-asm statement.
// This function computes the statement's operands: buffer descriptors and
// the per-lane LDS and memory offsets of the layouts below.

#include "fa_fwd_w64.inc"

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

// Raw buffer descriptor words (stride 0, bounds `bytes`): loads past the end
// return zero, stores past it are dropped.
__device__ __forceinline__ u32x4s raw_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4s{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Launch shape: 4 waves of 64 rows, 64-key tiles, a 4-stage ring of one K
// and one V tile (64 * 2d bytes each) per stage.
template <int D>
struct CfgW64 {
  static constexpr int BR = 256, BC = 64, NT = 256;
  static constexpr int ROWB = 2 * D;                // bytes per Q, K, V or O row
  static constexpr int KSTAGE = BC * ROWB;          // one K (or V) tile
  static constexpr int VRING = 4 * KSTAGE;          // the V ring follows the 4 K stages
  static constexpr int LDS_BYTES = 8 * KSTAGE;
  static constexpr int NPIECE = KSTAGE / 2048;      // 1 KiB DMA pieces per wave and stage
  static constexpr int NCH = ROWB / 16;             // 16-byte chunks per row
};


// One work item (batch b, query head hq, 256-row query tile qt): operands of
// the generated body, then the body itself.
template <typename T, bool CAUSAL, int D>
__device__ __forceinline__ void w64_item(const Params& p, uint32_t lds0, int b, int hq, int qt) {
  using C = CfgW64<D>;
  // The lane index through an opaque copy: the per-lane operands below are
  // then computed afresh for each item instead of being hoisted out of the
  // persistent loop, where they could only survive the body (which uses
  // nearly every vector register) in scratch memory.
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + 64 * wave;
  const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
  const size_t kvhead = (size_t)(b * p.Hkv + hkv) * p.Nkv;
  const u32x4s rq = raw_desc(static_cast<const uint16_t*>(p.q) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const u32x4s rk = raw_desc(static_cast<const uint16_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const u32x4s rv = raw_desc(static_cast<const uint16_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const u32x4s ro = raw_desc(static_cast<uint16_t*>(p.o) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const u32x4s rl = raw_desc(p.lse + qhead, (uint32_t)p.Nq * 4u);

  // DMA share: waves 0-1 move the K tile, waves 2-3 the V tile, NPIECE 1 KiB
  // pieces each (pieces ci0 .. ci0 + NPIECE-1 of the tile); piece c, lane l
  // writes 16 bytes of row c * (1024 / ROWB) + l / NCH at logical 16-byte
  // column l % NCH, stored at column (l % NCH) ^ swizzle(row).
  const bool isv = wave >= 2;
  const u32x4s rdma = isv ? rv : rk;
  const int ci0 = (C::NPIECE * wave) & (2 * C::NPIECE - 1);
  const uint32_t dmabase = lds0 + (isv ? (uint32_t)C::VRING : 0u) + (uint32_t)ci0 * 1024u;
  uint32_t dmaoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = (ci0 + u) * (1024 / C::ROWB) + lane / C::NCH;
    const int sw = isv ? swz_v<D>(row) : swz_k<D>(row);
    dmaoff[u] = (uint32_t)(row * C::ROWB + (((lane % C::NCH) ^ sw) * 16));
  }
  // K fragment (A operand of S^T = K Q^T): key row l32 of a 32-key block,
  // logical column 2cd + half, physical column ^ swizzle(row).
  const int swz = swz_k<D>(l32);
  const uint32_t kbase = (uint32_t)(l32 * C::ROWB + ((half ^ (swz & 1)) * 16) + ((swz >> 1) * 32));
  // V^T fragment (A operand of O^T += V^T P^T) by ds_read_b64_tr_b16: lane
  // (g, s) of its 16-lane group addresses key row 4*(g/2) + s/4 and 4
  // dimensions at 16*(g%2) + 4*(s%4); the read hands lane r of the group the
  // 4 keys of dimension 16*(g%2) + r.
  const int g16 = lane >> 4, s16 = lane & 15;
  const int vrow = (g16 >> 1) * 4 + (s16 >> 2);
  const uint32_t vbase = (uint32_t)(vrow * C::ROWB + swz_v<D>(vrow) * 16 + (g16 & 1) * 32 +
                                    ((s16 & 3) >> 1) * 16 + (s16 & 1) * 8);
  // (at d = 64 only kaddr0-3 and vaddr0-1 are operands of the body)
  const uint32_t kaddr0 = lds0 + (kbase ^ 0u), kaddr1 = lds0 + (kbase ^ 32u),
                 kaddr2 = lds0 + (kbase ^ 64u), kaddr3 = lds0 + (kbase ^ 96u),
                 kaddr4 = lds0 + (kbase ^ 128u), kaddr5 = lds0 + (kbase ^ 160u),
                 kaddr6 = lds0 + (kbase ^ 192u), kaddr7 = lds0 + (kbase ^ 224u);
  const uint32_t vr = lds0 + (uint32_t)C::VRING;
  const uint32_t vaddr0 = vr + (vbase ^ 0u), vaddr1 = vr + (vbase ^ 64u),
                 vaddr2 = vr + (vbase ^ 128u), vaddr3 = vr + (vbase ^ 192u);
  // Q rows q0w + 32h + l32, dimensions 16cd + 8*half (+ 32 rows for h = 1)
  const uint32_t qoff = (uint32_t)((q0w + l32) * C::ROWB + half * 16);
  // Mask limit: key j of row i is kept iff j <= min(N_kv - 1, causal ? i : inf)
  const int big = 0x3fffffff;
  const int lim0 = min(p.Nkv - 1, CAUSAL ? q0w + l32 : big);
  const int lim1 = min(p.Nkv - 1, CAUSAL ? q0w + 32 + l32 : big);
  // Epilogue: row q0w + (64 / NCH) i + lane / NCH, 16-byte column lane % NCH;
  // lse of row q0w + 32h + l32
  const uint32_t ooff = (uint32_t)((q0w + lane / C::NCH) * C::ROWB + (lane % C::NCH) * 16);
  const uint32_t lseoff = (uint32_t)((q0w + l32) * 4);
  const uint32_t obase = lds0 + (uint32_t)wave * (64u * C::ROWB);
  // Selector of the row-sum instruction (v_mfma_f32_16x16x32 reading P as B):
  // lane 16g + c holds A row c, columns 8g .. 8g+7; 1.0 in rows 0 and 8 for
  // g = 0, 2 and rows 4 and 12 for g = 1, 3, i.e. where lane % 8 == 4 * (g % 2).
  const uint32_t one2 = __is_same(T, __bf16) ? 0x3f803f80u : 0x3c003c00u;
  const uint32_t selv = ((lane & 7) == ((lane >> 2) & 4)) ? one2 : 0u;

  const int kv_end = CAUSAL ? min(p.Nkv, q0 + 256) : p.Nkv;
  const uint32_t ntiles = (uint32_t)((kv_end + 63) / 64);
  const uint32_t nmain = (uint32_t)(CAUSAL ? min((q0 + 1) / 64, p.Nkv / 64) : p.Nkv / 64);
  const uint32_t sl2 = __float_as_uint(p.sl2);
  const uint32_t qxor = p.qmode == 1 ? 0x80008000u : 0u;
  const uint32_t qand = p.qmode == 2 ? 0u : 0xffffffffu;

#define FA_W64_COMMON                                                                       \
  [rq] "s"(rq), [rdma] "s"(rdma), [ro] "s"(ro), [rl] "s"(rl), [dmabase] "s"(dmabase),       \
      [sl2] "s"(sl2), [qxor] "s"(qxor), [qand] "s"(qand), [ntiles] "s"(ntiles),             \
      [nmain] "s"(nmain), [obase] "s"(obase), [kaddr0] "v"(kaddr0), [kaddr1] "v"(kaddr1),  \
      [kaddr2] "v"(kaddr2), [kaddr3] "v"(kaddr3), [vaddr0] "v"(vaddr0), [vaddr1] "v"(vaddr1), \
      [dmaoff0] "v"(dmaoff[0]), [dmaoff1] "v"(dmaoff[1]), [dmaoff2] "v"(dmaoff[2]),         \
      [dmaoff3] "v"(dmaoff[3]), [qoff] "v"(qoff), [lim0] "v"(lim0), [lim1] "v"(lim1),       \
      [ooff] "v"(ooff), [lseoff] "v"(lseoff), [selv] "v"(selv)
#define FA_W64_OPERANDS                                                                     \
  FA_W64_COMMON, [kaddr4] "v"(kaddr4), [kaddr5] "v"(kaddr5), [kaddr6] "v"(kaddr6),          \
      [kaddr7] "v"(kaddr7), [vaddr2] "v"(vaddr2), [vaddr3] "v"(vaddr3)
  if constexpr (D == 128) {
    if constexpr (sizeof(T) == 2 && __is_same(T, __bf16)) {
      if constexpr (CAUSAL) asm volatile(FA_W64_BF16_CAUSAL : : FA_W64_OPERANDS : FA_W64_CLOBBERS);
      else asm volatile(FA_W64_BF16_FULL : : FA_W64_OPERANDS : FA_W64_CLOBBERS);
    } else {
      if constexpr (CAUSAL) asm volatile(FA_W64_F16_CAUSAL : : FA_W64_OPERANDS : FA_W64_CLOBBERS);
      else asm volatile(FA_W64_F16_FULL : : FA_W64_OPERANDS : FA_W64_CLOBBERS);
    }
  } else {
    if constexpr (sizeof(T) == 2 && __is_same(T, __bf16)) {
      if constexpr (CAUSAL) asm volatile(FA_W64D64_BF16_CAUSAL : : FA_W64_COMMON : FA_W64_CLOBBERS);
      else asm volatile(FA_W64D64_BF16_FULL : : FA_W64_COMMON : FA_W64_CLOBBERS);
    } else {
      if constexpr (CAUSAL) asm volatile(FA_W64D64_F16_CAUSAL : : FA_W64_COMMON : FA_W64_CLOBBERS);
      else asm volatile(FA_W64D64_F16_FULL : : FA_W64_COMMON : FA_W64_CLOBBERS);
    }
  }
#undef FA_W64_OPERANDS
#undef FA_W64_COMMON
}

// Non-causal grids: one work item per workgroup (map_block).  Causal grids
// are persistent: min(items, CUs) workgroups, all resident from the start,
// each taking the items of ranks bid, 2G - 1 - bid, 2G + bid, 4G - 1 - bid,
// ... (G workgroups; ranks in map_block's causal order, longest tiles
// first).  The zig-zag pairs long items with short ones, and no workgroup
// waits for the hardware to dispatch it: with one workgroup per CU the
// dispatcher hands new workgroups to the shader engines of an XCD in strict
// rotation and holds them while the next engine in turn has no free CU,
// which left CUs idle between short causal items.
template <typename T, bool CAUSAL, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_w64(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[CfgW64<D>::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_t*)lds;
  if constexpr (!CAUSAL) {
    int b, hq, qt;
    map_block(p, false, b, hq, qt);
    w64_item<T, false, D>(p, lds0, b, hq, qt);
  } else {
    const int G = (int)gridDim.x, bid = (int)blockIdx.x;
    const int n = p.n_heads * p.n_qtiles;
    for (int j = 0;; ++j) {
      const int r = (j & 1) ? (j + 1) * G - 1 - bid : j * G + bid;
      if (r >= n) break;   // every later rank of this workgroup is larger
      const int rr = r / p.n_heads;
      const int hl = r - rr * p.n_heads;
      const int b = hl / p.Hq;
      // the previous item's epilogue staged O in the LDS this item's
      // transfers overwrite
      if (j) __syncthreads();
      w64_item<T, true, D>(p, lds0, b, hl - b * p.Hq, p.n_qtiles - 1 - rr);
    }
  }
}

// ----------------------------------------------------- FP8 (e4m3) path
//
// The FlashAttention-3 direction the course page "FlashAttention:
// IO-aware attention kernel" (section 3.3) and the omica exam notes
// (section 4.5) name: the same exact tiled algorithm with 8-bit inputs on
// the matrix cores.  Q, K and V arrive as OCP E4M3 codes with one fp32
// dequantisation factor each.  The products run on
// v_mfma_f32_32x32x64_f8f6f4 (exact 8-bit products, fp32 accumulators):
// S^T = K Q^T contracts 64 head dimensions per instruction, and
// O^T += V^T P^T contracts the 64 keys of a whole tile in one instruction
// per 32 output dimensions, with P rounded to E4M3 (round to nearest even)
// on the way.  The row sums of that rounded P come from the matrix cores
// too (one more scaled 32x32x64 instruction per tile, with an all-ones
// operand), so O is a convex
// combination of V rows with the rounded weights, and the vector units do
// no additions for them.  Q's and K's factors fold into the exponent scale,
// V's into the final 1/l; O is written in bf16, lse in fp32.
//
// This compiled kernel (8 waves of 32 rows) serves head dimension 64; at 128
// the generated 64-row body above (attn_fwd_w64_e4m3) computes the same
// thing with the same layouts.  Workgroup, ring, DMA and lazy reference are
// those of the 16-bit path (256 rows, 64-key tiles, 4-stage ring).  The
// lazy reference moves past 2^8.  The unmasked tiles run as a ping-pong
// between the two halves of the workgroup (described at the loop).
//
// Operand layouts.  The 8-bit instruction pairs byte j of lane-half h of A
// with byte j of lane-half h of B, so both operands only need the same
// assignment of the contraction index to (lane-half, byte):
//   S:   lane-half h, byte j  <->  head dimension 64*cd + 32*h + j.  Q rows
//        sit in registers in that order; K rows are read from LDS as two
//        16-byte chunks.
//   P*V: lane-half h, byte j = 16*kt + r  <->  key 32*kt + 8*(r/4) + 4*h +
//        r%4, which is where the S accumulator leaves score r of 32-key block
//        kt.  P is packed straight from it, four bytes per dword.  V^T comes
//        from row-major V by four ds_read_b64_tr_b8 per 32 output columns:
//        within each group of 16 lanes the instruction hands result lane r,
//        byte t, the byte r%8 of what source lane 2t + r/8 addressed, so
//        source lane (t, r/8) of lane-group G addresses key row
//        16*i + 8*(t/4) + 4*(G/2) + t%4 (read i), head-dimension bytes
//        32*db + 16*(G%2) + 8*(r/8).
// Swizzles (XOR of the 16-byte chunk index within a row, period 16 rows)
// keep both reads free of bank conflicts: 16 rows reading one logical K
// chunk, and the 8 rows x 32 bytes of each half-wave of a V^T read, land on
// distinct banks.

template <int D>
struct Cfg8 {
  static constexpr int NW = 8;                  // waves per workgroup
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int BR = 32 * NW;            // query rows per workgroup
  static constexpr int BC = 64;                 // keys per K/V tile
  static constexpr int KT = BC / 32;            // 32-key blocks of S per tile
  static constexpr int STAGES = 4;              // LDS ring depth (tiles)
  static constexpr int ROWB = D;                // bytes per K/V row
  static constexpr int NCH = D / 16;            // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;       // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;      // K tile then V tile
  static constexpr int LDS_BYTES = STAGES * STAGEB;
  static constexpr int CHUNKS = STAGEB / 1024;  // 1 KiB DMA instructions per tile
  static constexpr int DPW = CHUNKS / NW;       // ... per wave
  static_assert(DPW * NW == CHUNKS && DPW >= 1, "DMA split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// K: 16 rows reading one logical chunk touch 16 distinct (bank line, chunk)
// pairs.  V: the XOR moves whole 32-byte blocks (bit 0 of the chunk index is
// kept), so that rows {0-3, 8-11} (or {4-7, 12-15}) hit distinct banks.
template <int D>
__device__ __forceinline__ int swz8_k(int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); }
template <int D>
__device__ __forceinline__ int swz8_v(int row) {
  return D == 128 ? ((((row >> 1) & 1) | (((row >> 3) & 1) << 1)) << 1) : (((row >> 3) & 1) << 1);
}

// The last result registers of the 8-bit 32x32x64 instruction are written 20
// issue slots after it, one more than the compiler pads before a vector
// read of them (measured on MI355X; the build's latency check rejects such a
// read).  A result is therefore handed to the rest of the code through this
// statement: it reads the result, so the compiler pads before it, and its own
// s_nop adds 5 slots the compiler counts as one.
__device__ __forceinline__ void settle(f32x16& x) { asm volatile("s_nop 4" : "+v"(x)); }

__device__ __forceinline__ f32x16 mma_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  // Format fields 0 (E4M3 for both operands), no block scales.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with block scales on B: lane c + 32b supplies the E8M0
// exponent (biased by 127, low byte of sb) of column c's block b of 32 K
// values, which are bytes 16b .. 16b+15 of both lane c and lane c + 32 (the
// instruction takes K from a lane pair in chunks of 16: measured on MI355X);
// A is unscaled (127).
__device__ __forceinline__ f32x16 mma_e4m3_bscaled(i32x8 a, i32x8 b, f32x16 c, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// -------------------------- 64 rows per wave, E4M3 inputs (head dimension 128)
//
// The FP8 forward on the generated 64-row body (gen_fwd_w64_fp8.py): the same
// computation as attn_fwd_e4m3 below (scores on the 8-bit instruction, each
// 64-key tile's probabilities rounded to E4M3 against a power-of-two reference
// of their own, carried by the P operand's block scales, row sums on the
// matrix instruction, O * V's factor / l in bf16), with each wave owning 64
// rows, one wave per SIMD, so that every K and V fragment read from LDS feeds
// two matrix instructions, and the instruction order set by the generator's
// issue-cost schedule.  Operand layouts are those of attn_fwd_e4m3 (same
// swizzles and byte orders); O leaves through LDS in whole bf16 rows.
struct CfgW64E {
  static constexpr int BR = 256, BC = 64, NT = 256;
  static constexpr int ROWB = 128;                  // bytes per E4M3 K or V row
  static constexpr int KSTAGE = BC * ROWB;
  static constexpr int VRING = 4 * KSTAGE;
  static constexpr int LDS_BYTES = 8 * KSTAGE;      // also holds the 4 waves' bf16 O tiles
  static constexpr int NPIECE = KSTAGE / 2048;
  static_assert(LDS_BYTES >= 4 * 64 * 256, "O staging");
};

template <bool CAUSAL>
__device__ __forceinline__ void w64_item_e4m3(const Params& p, uint32_t lds0, int b, int hq, int qt) {
  using C = CfgW64E;
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int q0w = q0 + 64 * wave;
  const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
  const size_t kvhead = (size_t)(b * p.Hkv + hkv) * p.Nkv;
  const u32x4s rq = raw_desc(static_cast<const uint8_t*>(p.q) + qhead * 128, (uint32_t)p.Nq * 128u);
  const u32x4s rk = raw_desc(static_cast<const uint8_t*>(p.k) + kvhead * 128, (uint32_t)p.Nkv * 128u);
  const u32x4s rv = raw_desc(static_cast<const uint8_t*>(p.v) + kvhead * 128, (uint32_t)p.Nkv * 128u);
  const u32x4s ro = raw_desc(static_cast<uint16_t*>(p.o) + qhead * 128, (uint32_t)p.Nq * 256u);
  const u32x4s rl = raw_desc(p.lse + qhead, (uint32_t)p.Nq * 4u);

  // DMA share: waves 0-1 the K tile, waves 2-3 the V tile, 4 KiB each; piece
  // c, lane l: 16 bytes of row 8c + l/8, logical chunk l%8 at chunk ^ swizzle.
  const bool isv = wave >= 2;
  const u32x4s rdma = isv ? rv : rk;
  const int ci0 = (C::NPIECE * wave) & (2 * C::NPIECE - 1);
  const uint32_t dmabase = lds0 + (isv ? (uint32_t)C::VRING : 0u) + (uint32_t)ci0 * 1024u;
  uint32_t dmaoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int row = (ci0 + u) * 8 + lane / 8;
    const int sw = isv ? swz8_v<128>(row) : swz8_k<128>(row);
    dmaoff[u] = (uint32_t)(row * C::ROWB + (((lane % 8) ^ sw) * 16));
  }
  // K fragment: key row l32, head-dimension bytes 64cd + 32*half as two chunks.
  const uint32_t kbase = (uint32_t)(l32 * C::ROWB + (((half * 2) ^ swz8_k<128>(l32)) * 16));
  const uint32_t kaddr0 = lds0 + (kbase ^ 0u), kaddr1 = lds0 + ((kbase ^ 0u) ^ 16u),
                 kaddr2 = lds0 + (kbase ^ 64u), kaddr3 = lds0 + ((kbase ^ 64u) ^ 16u);
  // V^T fragment by ds_read_b64_tr_b8 (the lane pattern of attn_fwd_e4m3).
  const int g16 = lane >> 4, s16 = lane & 15, t8 = s16 >> 1;
  const int vrow = (t8 >> 2) * 8 + (g16 >> 1) * 4 + (t8 & 3);
  const uint32_t vbase = (uint32_t)(vrow * C::ROWB + swz8_v<128>(vrow) * 16 + (g16 & 1) * 16 + (s16 & 1) * 8);
  const uint32_t vr = lds0 + (uint32_t)C::VRING;
  const uint32_t vaddr0 = vr + (vbase ^ 0u), vaddr1 = vr + (vbase ^ 32u),
                 vaddr2 = vr + (vbase ^ 64u), vaddr3 = vr + (vbase ^ 96u);
  // Q rows q0w + 32h + l32, bytes 64cd + 32*half (+ 32 rows for h = 1)
  const uint32_t qoff = (uint32_t)((q0w + l32) * C::ROWB + half * 32);
  const int big = 0x3fffffff;
  const int lim0 = min(p.Nkv - 1, CAUSAL ? q0w + l32 : big);
  const int lim1 = min(p.Nkv - 1, CAUSAL ? q0w + 32 + l32 : big);
  // bf16 O rows of 256 bytes: row q0w + 4i + lane/16, 16-byte column lane%16
  const uint32_t ooff = (uint32_t)((q0w + lane / 16) * 256 + (lane % 16) * 16);
  const uint32_t lseoff = (uint32_t)((q0w + l32) * 4);
  const uint32_t obase = lds0 + (uint32_t)wave * (64u * 256u);
  const int kv_end = CAUSAL ? min(p.Nkv, q0 + 256) : p.Nkv;
  const uint32_t ntiles = (uint32_t)((kv_end + 63) / 64);
  const uint32_t nmain = (uint32_t)(CAUSAL ? min((q0 + 1) / 64, p.Nkv / 64) : p.Nkv / 64);
  const uint32_t sl2 = __float_as_uint(p.sl2);
  const uint32_t qxor = p.qmode == 1 ? 0x80808080u : 0u;
  const uint32_t qand = p.qmode == 2 ? 0u : 0xffffffffu;
  const uint32_t oscale = __float_as_uint(p.oscale);

#define FA_W64_E4M3_OPERANDS                                                                \
  [rq] "s"(rq), [rdma] "s"(rdma), [ro] "s"(ro), [rl] "s"(rl), [dmabase] "s"(dmabase),       \
      [sl2] "s"(sl2), [qxor] "s"(qxor), [qand] "s"(qand), [ntiles] "s"(ntiles),             \
      [nmain] "s"(nmain), [obase] "s"(obase), [oscale] "s"(oscale), [kaddr0] "v"(kaddr0),   \
      [kaddr1] "v"(kaddr1), [kaddr2] "v"(kaddr2), [kaddr3] "v"(kaddr3), [vaddr0] "v"(vaddr0), \
      [vaddr1] "v"(vaddr1), [vaddr2] "v"(vaddr2), [vaddr3] "v"(vaddr3),                     \
      [dmaoff0] "v"(dmaoff[0]), [dmaoff1] "v"(dmaoff[1]), [dmaoff2] "v"(dmaoff[2]),         \
      [dmaoff3] "v"(dmaoff[3]), [qoff] "v"(qoff), [lim0] "v"(lim0), [lim1] "v"(lim1),       \
      [ooff] "v"(ooff), [lseoff] "v"(lseoff)
  if constexpr (CAUSAL) asm volatile(FA_W64_E4M3_CAUSAL : : FA_W64_E4M3_OPERANDS : FA_W64_CLOBBERS);
  else asm volatile(FA_W64_E4M3_FULL : : FA_W64_E4M3_OPERANDS : FA_W64_CLOBBERS);
#undef FA_W64_E4M3_OPERANDS
}

template <bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
attn_fwd_w64_e4m3(Params p) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[CfgW64E::LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_t*)lds;
  if constexpr (!CAUSAL) {
    int b, hq, qt;
    map_block(p, false, b, hq, qt);
    w64_item_e4m3<false>(p, lds0, b, hq, qt);
  } else {
    // persistent zig-zag grid, as attn_fwd_w64
    const int G = (int)gridDim.x, bid = (int)blockIdx.x;
    const int n = p.n_heads * p.n_qtiles;
    for (int j = 0;; ++j) {
      const int r = (j & 1) ? (j + 1) * G - 1 - bid : j * G + bid;
      if (r >= n) break;
      const int rr = r / p.n_heads;
      const int hl = r - rr * p.n_heads;
      const int b = hl / p.Hq;
      if (j) __syncthreads();
      w64_item_e4m3<true>(p, lds0, b, hl - b * p.Hq, p.n_qtiles - 1 - rr);
    }
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_e4m3_body(const Params& p) {
  using C = Cfg8<D>;
  constexpr int KT = C::KT;
  __shared__ __attribute__((aligned(1024))) unsigned char k0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k2[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k3[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v2[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v3[C::TILEB];
  auto kst = [&]<int S>() -> lds_t* {
    if constexpr ((S & 3) == 0) return (lds_t*)k0;
    else if constexpr ((S & 3) == 1) return (lds_t*)k1;
    else if constexpr ((S & 3) == 2) return (lds_t*)k2;
    else return (lds_t*)k3;
  };
  auto vst = [&]<int S>() -> lds_t* {
    if constexpr ((S & 3) == 0) return (lds_t*)v0;
    else if constexpr ((S & 3) == 1) return (lds_t*)v1;
    else if constexpr ((S & 3) == 2) return (lds_t*)v2;
    else return (lds_t*)v3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool second = wave >= C::NW / 2;   // the half of the workgroup that runs half a step behind
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int b, hq, qt;
  map_block(p, CAUSAL, b, hq, qt);
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * 32;        // first query row of this wave
  const int myq = qw0 + l32;             // this lane's query row

  const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
  const size_t kvhead = (size_t)(b * p.Hkv + hkv) * p.Nkv;
  const rsrc_t rq = make_rsrc(static_cast<const uint8_t*>(p.q) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const rsrc_t rk = make_rsrc(static_cast<const uint8_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rv = make_rsrc(static_cast<const uint8_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);

  const int kv_end = CAUSAL ? min(p.Nkv, q0 + C::BR) : p.Nkv;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  const int n_main = CAUSAL ? min((q0 + 1) / C::BC, p.Nkv / C::BC) : p.Nkv / C::BC;

  // Q operand first, so that waiting for it never waits for a K/V transfer.
  const uint32_t qxor = p.qmode == 1 ? 0x80808080u : 0u;
  const uint32_t qand = p.qmode == 2 ? 0u : 0xffffffffu;
  i32x8 qreg[D / 64];
#pragma unroll
  for (int cd = 0; cd < D / 64; ++cd) {
    const int off = myq * D + cd * 64 + half * 32;
    const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0));
    const u32x4 a = (lo ^ qxor) & qand, c = (hi ^ qxor) & qand;
    qreg[cd] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }

  // DMA of tile t into ring stage S (= t mod 4), DPW 1 KiB pieces per wave.
  auto issue = [&]<int S>(int t) {
    const int kv0 = t * C::BC;
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int i = wave * C::DPW + u;
      const bool isv = i >= C::CHUNKS / 2;
      const int ci = isv ? i - C::CHUNKS / 2 : i;
      const int slot = ci * 64 + lane;
      const int row = slot / C::NCH;
      const int c = (slot % C::NCH) ^ (isv ? swz8_v<D>(row) : swz8_k<D>(row));
      lds_t* dst = (isv ? vst.template operator()<S>() : kst.template operator()<S>()) + ci * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_t*)dst, 16,
                                               (kv0 + row) * C::ROWB + c * 16, 0, 0, 0);
    }
  };
  auto issue_any = [&](int t) {
    switch (t & 3) {
      case 0: issue.template operator()<0>(t); break;
      case 1: issue.template operator()<1>(t); break;
      case 2: issue.template operator()<2>(t); break;
      default: issue.template operator()<3>(t); break;
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int kbase = l32 * C::ROWB + (((half * 2) ^ swz8_k<D>(l32)) * 16);
  const int g16 = lane >> 4, s16 = lane & 15, t8 = s16 >> 1;
  const int vrow = (t8 >> 2) * 8 + (g16 >> 1) * 4 + (t8 & 3);
  const int vbase = vrow * C::ROWB + swz8_v<D>(vrow) * 16 + (g16 & 1) * 16 + (s16 & 1) * 8;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  // Row sums of the rounded P come from the matrix cores too: the P operand
  // (with its block scales) times an all-ones A, on the same instruction as
  // P*V; every row of the result holds the sum of its column's query, and
  // register 0 of lane l is the sum of query l % 32.
  f32x16 accs = f32x16{};
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  // held in its own 8 registers (as an opaque value, not rebuilt from one
  // register before every use)
  asm volatile("" : "+v"(ones));
  // Exponent references (log2 units).  O and the row sum are kept against
  // m_run, the same in both half-waves.  The probabilities of each tile are
  // formed against the tile's own m_tile = m_run - k, with k the integer
  // floor(m_run - tile maximum), so that the tile's largest probability lies
  // in (1/2, 1] (exactly 1 when the tile holds the reference's own score)
  // and the small ones keep E4M3's precision relative to their own tile
  // instead of falling below its subnormal range against a far larger key
  // elsewhere in the row.  The tile's factor 2^-k, a power of two, is applied
  // exactly by the matrix instructions as the E8M0 block scale sbyte of every
  // block of the P operand.
  float m_run = -INFINITY;
  float m_tile = 0.f;
  int sbyte = 127;

  auto compute_s = [&](const lds_t* st, f32x16 (&s)[KT]) {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) s[kt] = f32x16{};
#pragma unroll
    for (int cd = 0; cd < D / 64; ++cd) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int o = (kbase ^ (cd * 64)) + kt * 32 * C::ROWB;
        const u32x4 x0 = *(const u32x4 __attribute__((address_space(3)))*)(st + o);
        const u32x4 x1 = *(const u32x4 __attribute__((address_space(3)))*)(st + (o ^ 16));
        const i32x8 a = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        s[kt] = mma_e4m3(a, qreg[cd], s[kt]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) settle(s[kt]);
  };

  auto compute_pv = [&](const lds_t* st, const i32x8& pk) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const lds_t* a0 = st + (vbase ^ (db * 32));
      i32x2 r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(a0 + i * 16 * C::ROWB));
      const i32x8 x = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
      acc[db] = mma_e4m3_bscaled(x, pk, acc[db], sbyte);
    }
    accs = mma_e4m3_bscaled(ones, pk, accs, sbyte);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) settle(acc[db]);
    settle(accs);
  };

  // New exponent reference from a tile of raw scores; O and the sum move to
  // it (only when it moves: lazy reference).
  auto rebase = [&](const f32x16 (&s)[KT]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = pair_max(mx);
    const float mc = mx * p.sl2;
    const float m_new = (mc > m_run + kLazy) ? mc : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    // k >= -kLazy; a tile more than 200 below the reference (or with no
    // allowed key) is formed against m_run - 200 and scaled by byte 0: its
    // weight, under 2^-127 of the row's, is dropped.  No finite score yet:
    // P = 0 against reference 0.
    const float k = fminf(floorf(m_run - mc), 200.f);
    m_tile = m_run == -INFINITY ? 0.f : m_run - k;
    sbyte = (int)fmaxf(127.f - k, 0.f);
    accs[0] *= alpha;
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
    }
  };

  // P = exp2(s * sl2 - m_tile), rounded to E4M3 in the byte order of the P*V operand.
  auto exponentiate = [&](const f32x16 (&s)[KT], i32x8& pk) {
    const float mu = m_tile;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float e0 = fast_exp2(fmaf(s[kt][4 * w], p.sl2, -mu));
        const float e1 = fast_exp2(fmaf(s[kt][4 * w + 1], p.sl2, -mu));
        const float e2 = fast_exp2(fmaf(s[kt][4 * w + 2], p.sl2, -mu));
        const float e3 = fast_exp2(fmaf(s[kt][4 * w + 3], p.sl2, -mu));
        // The first conversion's upper half is rewritten by the second, so
        // its pass-through operand can be any register: e0's own, which dies
        // here (no extra move).
        int d = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, __float_as_int(e0), false);
        d = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, d, true);
        pk[kt * 4 + w] = d;
      }
    }
  };

  f32x16 s[KT];
  i32x8 pk;

  issue.template operator()<0>(0);
  if (n_tiles > 1) issue.template operator()<1>(1);
  if (n_tiles > 2) issue.template operator()<2>(2);

  // Unmasked tiles.  Per tile j a wave runs a matrix-core phase G(j)
  // (O += V_j P_j, then S_{j+1} = K_{j+1} Q^T) and a vector phase X(j)
  // (reference and P_{j+1} from S_{j+1}), separated by workgroup barriers.
  // The second half of the workgroup runs the same code one barrier later,
  // so each SIMD holds one wave in G while its other wave is in X (the
  // ping-pong of FlashAttention-3):
  //   first half:   X(-1) | G(0) ... X(0) | G(1) ... X(1) | ...
  //   second half:  X(-1) ......... | G(0) ... X(0) | G(1) ... X(1) | ...
  // Tile k+3 is issued at the start of step k into the stage of tile k-1,
  // whose last reader (the second half's G(k-1)) finished one barrier earlier.
  if (n_main > 0) {
    if (n_tiles > 2) wait_vm_lgkm<C::DPW>();
    else wait_vm_lgkm<0>();
    barrier();
    compute_s(kst.template operator()<0>(), s);
    rebase(s);
    exponentiate(s, pk);
    if (second) barrier();
    auto step = [&]<int R>(int k) {
      if (k + 3 < n_tiles) issue.template operator()<(R + 3) & 3>(k + 3);
      compute_pv(vst.template operator()<R>(), pk);
      compute_s(kst.template operator()<(R + 1) & 3>(), s);
      if (k + 3 < n_tiles) wait_vm_lgkm<C::DPW>();   // tile k+2 has landed
      else wait_vm_lgkm<0>();
      barrier();
      // Keep each phase's work between its barriers: the scores count as
      // produced here (no max hoisted above), P as consumed (no exp sunk below).
      asm volatile("" : "+v"(s[0]), "+v"(s[1]));
      rebase(s);
      exponentiate(s, pk);
      asm volatile("" : "+v"(pk));
      barrier();
    };
    int k = 0;
    for (; k + 4 <= n_main - 1; k += 4) {
      step.template operator()<0>(k);
      step.template operator()<1>(k + 1);
      step.template operator()<2>(k + 2);
      step.template operator()<3>(k + 3);
    }
    for (; k < n_main - 1; ++k) {
      switch (k & 3) {
        case 0: step.template operator()<0>(k); break;
        case 1: step.template operator()<1>(k); break;
        case 2: step.template operator()<2>(k); break;
        default: step.template operator()<3>(k); break;
      }
    }
    switch ((n_main - 1) & 3) {
      case 0: compute_pv(vst.template operator()<0>(), pk); break;
      case 1: compute_pv(vst.template operator()<1>(), pk); break;
      case 2: compute_pv(vst.template operator()<2>(), pk); break;
      default: compute_pv(vst.template operator()<3>(), pk); break;
    }
    if (!second) barrier();
  }

  // Masked tiles (ragged tail, causal diagonal): one tile at a time, every
  // wave in step.  Tiles up to max(2, n_main + 1) were issued above.
  const int issued = max(2, n_main + 1);
  for (int t = n_main; t < n_tiles; ++t) {
    if (t > issued) issue_any(t);
    wait_vm_lgkm<0>();
    barrier();
    const int kv0 = t * C::BC;
    const bool active = (qw0 < p.Nq) && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      auto body = [&]<int R>() {
        compute_s(kst.template operator()<R>(), s);
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            if ((key >= p.Nkv) || (CAUSAL && key > myq)) s[kt][r] = -INFINITY;
          }
        }
        rebase(s);
        exponentiate(s, pk);
        compute_pv(vst.template operator()<R>(), pk);
      };
      switch (t & 3) {
        case 0: body.template operator()<0>(); break;
        case 1: body.template operator()<1>(); break;
        case 2: body.template operator()<2>(); break;
        default: body.template operator()<3>(); break;
      }
    }
    barrier();
  }

  // Epilogue: O = acc * (V's factor / l) in bf16, lse in fp32.
  const rsrc_t ro = make_rsrc(static_cast<uint16_t*>(p.o) + qhead * D, (uint32_t)p.Nq * D * 2u);
  const rsrc_t rl = make_rsrc(p.lse + qhead, (uint32_t)p.Nq * 4u);
  const float l_tot = accs[0];
  const float inv = p.oscale / l_tot;
  using M = Mma16<__bf16>;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = M::pack(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
      w[1] = M::pack(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, w), ro,
                                            (myq * D + db * 32 + g * 8 + half * 4) * 2, 0, 0);
    }
  }
  if (half == 0)
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((m_run + fast_log2(l_tot)) * kLn2), rl,
                                          myq * 4, 0, 0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(Cfg8<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_e4m3(Params p) {
  attn_fwd_e4m3_body<D, CAUSAL>(p);
}

// --------------------------------------------------- split-KV (16-bit) path
//
// For shapes with few query rows per key/value head (decoding: N_q = 1), the
// 256-row workgroup above would leave almost every MFMA row empty and the GPU
// mostly idle.  The course page "FlashAttention: IO-aware attention kernel"
// (section 3, where the method helps and where it does not) names the decode
// variant, FlashDecoding, that parallelises over the key/value length
// instead.  This path cuts the key sequence of every (batch, key/value head)
// into num_splits chunks and gives each (row block, chunk) pair to one wave.  A row block is 32 consecutive "packed" rows of one key/value head:
// packed row r stands for query head g*G + r / N_q and query row r % N_q
// (G = Hq / Hkv), so the query heads that share a K/V head share its
// stream, and a decode step of a 7:1 group fills 7 MFMA rows instead of 1.
// Each wave keeps its own running reference, sum and accumulator over its
// chunk (the same recurrence and lazy reference as the main path), and
// writes the chunk's normalised output and its lse in fp32 to a workspace.
// A second kernel merges the chunks of every row with the block merge rule
// of the omica exam notes (section 2.3), in its form for normalised
// partials: each chunk weighted by exp(lse_s - lse).
//
// Waves are independent (no barrier).  Each streams its chunk in tiles of
// 32 keys: the K fragments go straight from global memory into registers
// (each lane reads its own key row), double-buffered one tile ahead; V goes
// by DMA into a private two-stage LDS ring, one tile ahead, and is read
// transposed like in the main path.  Eight waves per workgroup (two per
// SIMD) keep every MFMA within 256 registers in its VGPR form.

template <int D>
struct CfgSplit {
  static constexpr int NW = 8;                  // waves (work items) per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int BC = 32;                 // keys per tile
  static constexpr int ROWB = D * 2;            // bytes per K/V row
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;       // one V tile of one wave
  static constexpr int VPT = TILEB / 1024;      // 1 KiB DMA instructions per V tile
  static constexpr int KPT = D / 16;            // K fragment loads per tile
  static constexpr int LDS_BYTES = 2 * NW * TILEB;
  static_assert(VPT >= 1, "DMA split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

struct SplitParams {
  const void* q;
  const void* k;
  const void* v;
  float* ows;       // [S][B*Hq*N_q][d] chunk outputs, normalised
  float* lws;       // [S][B*Hq*N_q]    chunk lse (natural log), -inf when empty
  int B, Hq, Hkv, Nq, Nkv;
  int group;        // G = Hq / Hkv
  int R;            // packed rows per (b, kv head) = G * N_q
  int nrb;          // row blocks per (b, kv head) = ceil(R / 32)
  int S;            // chunks per row block (chunk s: tiles s, s+S, s+2S, ...)
  long long items;  // B * Hkv * nrb * S
  long long rows;   // B * Hq * N_q
  float sl2;
  int qmode;
  // Paged K/V only (k and v then point at the block pools):
  const int* btab;     // [B][mbps] pool block of each run of 2^lbs keys of a sequence
  const int* seqlens;  // [B] keys held for each sequence
  int mbps;            // block-table row length
  int lbs;             // log2 of the keys per block
  int nblocks;         // blocks in each pool
  uint32_t pool_bytes; // bytes of each pool
};

template <typename T, int D, bool CAUSAL, bool PAGED>
__device__ __forceinline__ void attn_splitkv_body(const SplitParams& p) {
  using C = CfgSplit<D>;
  using M = Mma16<T>;
  __shared__ __attribute__((aligned(1024))) unsigned char v0[C::NW * C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[C::NW * C::TILEB];
  auto vst = [&]<int S>() -> lds_t* { if constexpr ((S & 1) == 0) return (lds_t*)v0; else return (lds_t*)v1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const long long item = (long long)blockIdx.x * C::NW + wave;
  if (item >= p.items) return;   // no barrier in this kernel: idle waves may leave
  // Dense: the chunks of one (batch, key/value head) are neighbours.  Paged:
  // the key/value heads are fastest, so that the waves reading the pieces of
  // one token row of a pool block (one per head) run side by side.
  int s, rb, g, b;
  if constexpr (PAGED) {
    g = (int)(item % p.Hkv);
    long long rest = item / p.Hkv;
    s = (int)(rest % p.S);
    rest /= p.S;
    rb = (int)(rest % p.nrb);
    b = (int)(rest / p.nrb);
  } else {
    s = (int)(item % p.S);
    long long rest = item / p.S;
    rb = (int)(rest % p.nrb);
    rest /= p.nrb;
    g = (int)(rest % p.Hkv);
    b = (int)(rest / p.Hkv);
  }

  // This lane's packed row, its query head and query index.
  const int r = rb * 32 + l32;
  const bool row_ok = r < p.R;
  const int rr = row_ok ? r : p.R - 1;
  const int hq = g * p.group + rr / p.Nq;
  const int qi = rr - (rr / p.Nq) * p.Nq;
  // Largest and smallest query index among the block's rows (causal limits).
  const int r_lo = rb * 32, r_hi = min(rb * 32 + 31, p.R - 1);
  const bool one_head = (r_lo / p.Nq) == (r_hi / p.Nq);
  const int qi_max = one_head ? r_hi % p.Nq : p.Nq - 1;
  const int qi_min = one_head ? r_lo % p.Nq : 0;

  // Chunk s owns the 32-key tiles s, s + S, s + 2S, ... of the keys any row
  // of the block may see.  Interleaving (rather than one contiguous range
  // per chunk) makes the S waves of one head read neighbouring tiles at the
  // same time, so the memory traffic of all waves stays close to a few
  // sequential streams instead of thousands of streams with equal address
  // strides, which collide in the same memory channels.
  // Keys of this (batch, key/value head), and the causal offset: query i
  // sees key j iff j <= i + coff (0 for the dense layout; the paged layout
  // aligns the N_q queries with the last N_q keys of the sequence).
  int nkv = p.Nkv, coff = 0;
  if constexpr (PAGED) {
    nkv = min(max(p.seqlens[b], 0), p.mbps << p.lbs);
    coff = nkv - p.Nq;
  }
  int c1 = nkv;                                                  // one past the last key used
  if (CAUSAL) c1 = min(c1, qi_max + coff + 1);
  const int t_all = c1 > 0 ? (c1 + C::BC - 1) / C::BC : 0;
  const int n_tiles = s < t_all ? (t_all - s + p.S - 1) / p.S : 0;
  // Dense layout: each (batch, key/value head) starts its sequence of tiles
  // at a different position (and wraps around).  The heads' K/V blocks are
  // equally aligned, so without it all heads would stream the same offsets
  // at the same time.  The paged layout keeps the plain order: the key/value
  // heads of a sequence share each pool block, and reading it together is
  // faster.
  const int rot = (n_tiles > 0 && !PAGED) ? (b * p.Hkv + g) % n_tiles : 0;
  auto tile_key0 = [&](int t) {
    int u = t + rot;
    u -= (u >= n_tiles) ? n_tiles : 0;
    return (s + u * p.S) * C::BC;
  };

  const size_t kvhead = (size_t)(b * p.Hkv + g) * p.Nkv;
  const rsrc_t rk = PAGED ? make_rsrc(p.k, p.pool_bytes)
                          : make_rsrc(static_cast<const uint16_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rv = PAGED ? make_rsrc(p.v, p.pool_bytes)
                          : make_rsrc(static_cast<const uint16_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);

  // Byte offset of key `key` of tile t in K or V.  Dense: row `key` of the
  // head.  Paged: the block table maps key run key >> lbs of the sequence to
  // a pool block, whose rows hold [token][Hkv][d]; a 32-key tile touches at
  // most two blocks (2^lbs >= 16), looked up once per tile with scalar loads.
  // Keys past the sequence (last tile) re-read its last key and are masked;
  // block numbers are clamped into the pool, so a bad table entry cannot
  // send a load outside it.
  struct TileMap {
    int key0, blk0, id0, id1;
  };
  auto tile_map = [&](int t) -> TileMap {
    TileMap m{tile_key0(t), 0, 0, 0};
    if constexpr (PAGED) {
      // Constant address space: the compiler reads the (wave-uniform) entries with scalar loads.
      const __attribute__((address_space(4))) int* tab =
          (const __attribute__((address_space(4))) int*)(uintptr_t)p.btab + (size_t)b * p.mbps;
      const int last = nkv - 1;
      m.blk0 = m.key0 >> p.lbs;
      m.id0 = min(max(tab[m.blk0], 0), p.nblocks - 1);
      m.id1 = min(max(tab[min(m.key0 + 16, last) >> p.lbs], 0), p.nblocks - 1);
    }
    return m;
  };
  auto key_off = [&](const TileMap& m, int r) -> uint32_t {
    if constexpr (PAGED) {
      const int key = min(m.key0 + r, nkv - 1);
      const int id = (key >> p.lbs) == m.blk0 ? m.id0 : m.id1;
      return ((uint32_t)(id << p.lbs) + (uint32_t)(key & ((1 << p.lbs) - 1))) *
                 (uint32_t)(p.Hkv * C::ROWB) + (uint32_t)(g * C::ROWB);
    } else {
      return (uint32_t)(m.key0 + r) * C::ROWB;
    }
  };

  // K fragments of tile t: lane (l32, half) holds key tile_key0(t) + l32, dims
  // cd*16 + half*8 .. +7 (dense rows past N_kv read as zeros).
  auto load_k = [&](const TileMap& m, u32x4 (&kr)[C::KPT]) {
    const uint32_t off = key_off(m, l32) + half * 16;
#pragma unroll
    for (int cd = 0; cd < C::KPT; ++cd)
      kr[cd] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off + cd * 32, 0, 0));
  };
  // DMA of the V rows of tile t into this wave's part of ring stage S.
  auto issue_v = [&]<int S>(const TileMap& m) {
#pragma unroll
    for (int u = 0; u < C::VPT; ++u) {
      const int slot = u * 64 + lane;
      const int row = slot / C::NCH;
      const int c = (slot % C::NCH) ^ swz_v<D>(row);
      lds_t* dst = vst.template operator()<S>() + wave * C::TILEB + u * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dst, 16, key_off(m, row) + c * 16, 0, 0, 0);
    }
  };

  u32x4 ka[C::KPT], kb[C::KPT];
  if (n_tiles > 0) {
    const TileMap m0 = tile_map(0);
    load_k(m0, ka);
    issue_v.template operator()<0>(m0);
  }

  // Q^T operand of the wave's 32 packed rows (zeros past R).
  const uint32_t qxor = p.qmode == 1 ? 0x80008000u : 0u;
  const uint32_t qand = p.qmode == 2 ? 0u : 0xffffffffu;
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((size_t)(b * p.Hq + hq) * p.Nq + qi) * D;
  u32x4 qreg[D / 16];
#pragma unroll
  for (int cd = 0; cd < D / 16; ++cd) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row_ok) x = *reinterpret_cast<const u32x4*>(qrow + cd * 16 + half * 8);
    qreg[cd] = (x ^ qxor) & qand;
  }

  const int g16 = lane >> 4, s16 = lane & 15;
  const int vrow = (g16 >> 1) * 4 + (s16 >> 2);
  const int vbase = vrow * C::ROWB + (swz_v<D>(vrow) >> 2) * 64 + (g16 & 1) * 32 +
                    ((s16 & 3) >> 1) * 16 + (s16 & 1) * 8;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Tile t from K registers kc and V stage S.  Inside the loop every step
  // prefetches tile t+1 into kn and stage S^1; the last tile of the loop
  // "prefetches" itself again (a cached re-read), so the loop body has no
  // branch around its memory operations and the wait count is exact.  The
  // peeled final step (LAST) prefetches nothing and waits for everything: a
  // prefetch there would load registers nobody reads, which the compiler may
  // drop, and a fixed wait count would then be wrong.
  auto step = [&]<int S, bool LAST>(int t, u32x4 (&kc)[C::KPT], u32x4 (&kn)[C::KPT]) {
    if constexpr (LAST) {
      (void)kn;
      wait_vm_lgkm<0>();
    } else {
      const TileMap mn = tile_map(min(t + 1, n_tiles - 1));
      load_k(mn, kn);
      issue_v.template operator()<S ^ 1>(mn);
      wait_vm_lgkm<C::KPT + C::VPT>();
    }
    f32x16 sc = f32x16{};
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) sc = M::mma(kc[cd], qreg[cd], sc);
    const int kv0 = tile_key0(t);
    const bool need_mask = (kv0 + C::BC > c1) || (CAUSAL && kv0 + C::BC - 1 > qi_min + coff);
    if (need_mask) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kv0 + (e >> 2) * 8 + half * 4 + (e & 3);
        if (key >= c1 || (CAUSAL && key > qi + coff)) sc[e] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = pair_max(mx);
    const float mc = mx * p.sl2;
    const float m_new = (mc > m_run + kLazy) ? mc : m_run;
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if (wave_any(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    u32x4 pk[2];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float e0 = fast_exp2(fmaf(sc[cc * 8 + 2 * w], p.sl2, -mu));
        const float e1 = fast_exp2(fmaf(sc[cc * 8 + 2 * w + 1], p.sl2, -mu));
        const uint32_t pr = M::pack(e0, e1);
        pk[cc][w] = pr;
        if (w & 1) ls1 = M::sum2(pr, ls1);
        else ls0 = M::sum2(pr, ls0);
      }
    }
    l_run += ls0 + ls1;
    // The empty asm makes the compiler recompute the few XORs below every
    // tile instead of keeping one address register per (stage, fragment).
    int vb = wave * C::TILEB + vbase;
    asm volatile("" : "+v"(vb));
    const lds_t* vs = vst.template operator()<S>();
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const lds_t* a0 = vs + (vb ^ (db * 64)) + (cc * 16) * C::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a0);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(a0 + 8 * C::ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 x = {l2[0], l2[1], h2[0], h2[1]};
        acc[db] = M::mma(x, pk[cc], acc[db]);
      }
    }
  };
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    step.template operator()<0, false>(t, ka, kb);
    step.template operator()<1, false>(t + 1, kb, ka);
  }
  if (t < n_tiles) step.template operator()<0, true>(t, ka, kb);

  // Chunk result: normalised output and lse, or (0, -inf) for an empty chunk.
  const float l_tot = pair_sum(l_run);
  const bool has = l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
  if (row_ok) {
    const size_t row = (size_t)(b * p.Hq + hq) * p.Nq + qi;
    float* dst = p.ows + ((size_t)s * p.rows + row) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 w = {acc[db][4 * gq] * inv, acc[db][4 * gq + 1] * inv, acc[db][4 * gq + 2] * inv,
                         acc[db][4 * gq + 3] * inv};
        *reinterpret_cast<f32x4*>(dst + db * 32 + gq * 8 + half * 4) = w;
      }
    }
    if (half == 0) p.lws[(size_t)s * p.rows + row] = has ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D, bool CAUSAL, bool PAGED>
__global__ void __launch_bounds__(CfgSplit<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_splitkv_mfma16(SplitParams p) {
  attn_splitkv_body<T, D, CAUSAL, PAGED>(p);
}

// Merge of the chunk results of every row: lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s, rounded once to the output type.  One
// workgroup per row.  The kernel is a chain of dependent steps on a small
// amount of data, so its time is latency: the chunk partials are loaded
// before the weights are known (they do not depend on them), the max and
// the sum of the weights are wave butterflies with one barrier each, then
// G groups of D/4 threads (4 head dimensions each) sum a strided subset of
// the chunks and LDS adds the G partial sums.
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_splitkv_combine(const float* __restrict__ ows,
                                                             const float* __restrict__ lws,
                                                             T* __restrict__ o, float* __restrict__ lse,
                                                             long long rows, int S) {
  constexpr int LPR = D / 4;            // threads per dimension sweep
  constexpr int G = 256 / LPR;          // chunk groups
  constexpr int PRE = 8;                // chunk partials per thread loaded ahead of the weights
  __shared__ float w_s[FA_SPLITKV_MAX_SPLITS];
  __shared__ float red[2][4];
  __shared__ f32x4 part[G][LPR];
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv_id = tid >> 6;
  const int c = tid % LPR, grp = tid / LPR;

  // Every load that does not depend on the weights is issued first: this
  // thread's chunk lse and its first PRE chunk partials.
  const float lv = tid < S ? lws[(size_t)tid * rows + row] : -INFINITY;
  f32x4 pre[PRE];
#pragma unroll
  for (int u = 0; u < PRE; ++u) {
    const int s = grp + u * G;
    pre[u] = s < S ? *reinterpret_cast<const f32x4*>(ows + ((size_t)s * rows + row) * D + c * 4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Largest chunk lse: a butterfly within each wave, then the four waves.
  float m = lv;
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) m = fmaxf(m, __shfl_xor(m, w));
  if ((tid & 63) == 0) red[0][wv_id] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  // Weights exp(lse_s - max); empty chunks (lse_s = -inf) get 0.
  const float wv = (tid < S && lv != -INFINITY) ? fast_exp2((lv - mx) * kLog2e) : 0.f;
  if (tid < S) w_s[tid] = wv;
  float sm = wv;
#pragma unroll
  for (int w = 32; w > 0; w >>= 1) sm += __shfl_xor(sm, w);
  if ((tid & 63) == 0) red[1][wv_id] = sm;
  __syncthreads();
  const float wsum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < PRE; ++u) {
    const int s = grp + u * G;
    if (s < S) {
      const float w = w_s[s];
      if (w != 0.f) acc += w * pre[u];
    }
  }
  for (int s = grp + PRE * G; s < S; s += G) {
    const float w = w_s[s];
    if (w != 0.f) acc += w * *reinterpret_cast<const f32x4*>(ows + ((size_t)s * rows + row) * D + c * 4);
  }
  part[grp][c] = acc;
  __syncthreads();
  if (tid < LPR) {
    f32x4 t = part[0][tid];
#pragma unroll
    for (int g2 = 1; g2 < G; ++g2) t += part[g2][tid];
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;   // a row with no key at all: O = 0, lse = -inf
    T out4[4] = {(T)(t[0] * inv), (T)(t[1] * inv), (T)(t[2] * inv), (T)(t[3] * inv)};
    *reinterpret_cast<u32x2*>(o + row * D + tid * 4) = __builtin_bit_cast(u32x2, out4);
    if (tid == 0) lse[row] = mx + fast_log2(wsum) * kLn2;
  }
}

// ------------------------------------------------------ backward (16-bit)
//
// Recomputation, as the kyonqi walkthrough ("Flash Attention Backward") and
// the omica exam notes (section 2.5) describe it: the forward keeps O and one
// statistic per row (lse), and the backward forms S and P again tile by tile
// from Q, K and lse, P = exp(scale * q.k - lse), never storing either.  The
// gradients are those of O = softmax(S) V for the scalar sum(O * dO):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = scale dS K,  dK = scale dS^T Q,
// with dK, dV of a key/value head summed over its query heads.  Three
// launches: a row pass writing (lse * log2 e, D) per query row to the
// workspace, a key-stationary pass for dK and dV, and a query-stationary pass
// for dQ.  Every output element is written once by one wave (no atomics), so
// the result is deterministic.
//
// Tiles live in LDS with the two-way swizzle swz_kt (16-byte chunk index XOR a
// row function); the same layout serves both operand reads, the 16-byte row
// reads and the transposed ds_read_b64_tr_b16 reads, without bank conflicts.

// Transposed-read lane base for rows vrow and vrow + 8 of a 16-row group
// stored with swz_kt; the head-dimension block db is applied as "^ (db * 64)".
template <int D>
__device__ __forceinline__ int tr_base_bwd(int lane, int hi) {
  constexpr int ROWB = D * 2;
  const int g16 = lane >> 4, s16 = lane & 15;
  const int row = (g16 >> 1) * 4 + (s16 >> 2) + 8 * hi;
  const int c = (g16 & 1) * 2 + ((s16 & 3) >> 1);
  return row * ROWB + ((c ^ swz_kt<D>(row)) * 16) + (s16 & 1) * 8;
}

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float2* stats;    // [B*Hq*N_q]: (lse * log2 e, rowsum(dO * O))
  float* part;      // [hsplit][2][B*Hkv*N_kv*d] fp32 partial dK, dV (hsplit > 1 only)
  int B, Hq, Hkv, Nq, Nkv;
  int group;
  float scale;      // as given (any finite value)
  float sl2;        // scale * log2 e (sign kept)
  int n_tiles;      // workgroup tiles along the stationary axis
  int items;        // work items of the kernel launched with these parameters
  int hsplit;       // dK/dV pass: query heads of a group dealt over this many workgroups
};

// Row pass: stats[row] = (lse * log2 e, sum_d dO[row][d] * O[row][d]).
template <typename T, int D>
__global__ void __launch_bounds__(256) attn_bwd_prep(BwdParams p, long long rows) {
  constexpr int LPR = D / 8;               // lanes per row, 8 elements each
  const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  const bool ok = row < rows;
  const long long r = ok ? row : 0;
  float acc = 0.f;
  if (ok) {
    const u32x4 a = *(reinterpret_cast<const u32x4*>(static_cast<const T*>(p.dout) + r * D) + part);
    const u32x4 b = *(reinterpret_cast<const u32x4*>(static_cast<const T*>(p.o) + r * D) + part);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = Mma16<T>::dot2(a[i], b[i], acc);
  }
#pragma unroll
  for (int w = LPR / 2; w > 0; w >>= 1) acc += __shfl_xor(acc, w);
  if (ok && part == 0) p.stats[r] = make_float2(p.lse[r] * kLog2e, acc);
}

template <int D>
struct CfgBwdKV {
  static constexpr int NW = 8;                  // waves; 32 keys each
  static constexpr int NT = 64 * NW;
  static constexpr int BKV = 32 * NW;           // keys per workgroup
  static constexpr int BQ = 32;                 // query rows per step
  static constexpr int ROWB = D * 2;
  static constexpr int NCH = D / 8;
  static constexpr int QTB = BQ * ROWB;         // one Q (or dO) step tile
  static constexpr int CH = QTB / 1024;         // 1 KiB DMA chunks per step tile
  static constexpr int DPW = 2 * CH / NW;       // Q + dO chunks per wave per step
  static constexpr int VCH = BKV * ROWB / 1024; // V chunks (once)
  static_assert(DPW >= 1 && DPW * NW == 2 * CH, "DMA split");
};

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dkdv_body(const BwdParams& p, int item, int n_items) {
  using C = CfgBwdKV<D>;
  using M = Mma16<T>;
  __shared__ __attribute__((aligned(1024))) unsigned char q0s[C::QTB];
  __shared__ __attribute__((aligned(1024))) unsigned char q1s[C::QTB];
  __shared__ __attribute__((aligned(1024))) unsigned char o0s[C::QTB];
  __shared__ __attribute__((aligned(1024))) unsigned char o1s[C::QTB];
  __shared__ __attribute__((aligned(256))) unsigned char st0[C::BQ * 8];
  __shared__ __attribute__((aligned(256))) unsigned char st1[C::BQ * 8];
  __shared__ __attribute__((aligned(1024))) unsigned char vall[C::BKV * C::ROWB];
  auto qst = [&]<int S>() -> lds_t* { if constexpr ((S & 1) == 0) return (lds_t*)q0s; else return (lds_t*)q1s; };
  auto ost = [&]<int S>() -> lds_t* { if constexpr ((S & 1) == 0) return (lds_t*)o0s; else return (lds_t*)o1s; };
  auto sst = [&]<int S>() -> lds_t* { if constexpr ((S & 1) == 0) return (lds_t*)st0; else return (lds_t*)st1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Work item: (b, kv head, head share, key tile).  Head share hs takes the
  // query heads hs, hs + hsplit, ... of the group.  Non-causal: key tiles
  // fastest.  Causal: the first key tiles see the most queries, so they are
  // listed first, (b, kv head, share) fastest, and the longest items start in
  // the first round of workgroups.
  const int n_r1 = n_items / p.n_tiles;
  const int xl = xcd_local(item, n_items);
  const int kt = CAUSAL ? item / n_r1 : xl % p.n_tiles;
  const int r1 = CAUSAL ? item % n_r1 : xl / p.n_tiles;
  const int hs = r1 % p.hsplit;
  const int bg = r1 / p.hsplit;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int n_heads = (p.group - hs + p.hsplit - 1) / p.hsplit;
  const int k0 = kt * C::BKV;
  const int kw0 = k0 + wave * 32;               // this wave's first key
  const int key = kw0 + l32;                    // this lane's key (column of S)

  const size_t kvhead = (size_t)(b * p.Hkv + g) * p.Nkv;
  const rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);

  // V rows of the whole key tile into LDS, once.
#pragma unroll
  for (int u = 0; u < C::VCH / C::NW; ++u) {
    const int ci = wave * (C::VCH / C::NW) + u;
    const int slot = ci * 64 + lane;
    const int row = slot / C::NCH;
    const int c = (slot % C::NCH) ^ swz_kt<D>(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_t*)vall + ci * 1024, 16,
                                             (k0 + row) * C::ROWB + c * 16, 0, 0, 0);
  }
  // K^T operand of the wave's 32 keys, in registers for the whole pass.
  u32x4 kreg[D / 16];
#pragma unroll
  for (int cd = 0; cd < D / 16; ++cd)
    kreg[cd] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rk, key * C::ROWB + cd * 32 + half * 16, 0, 0));

  // Query steps: every query head of the group, query rows from the first
  // one that can see this key tile (causal) to N_q.
  const int qs0 = CAUSAL ? k0 / C::BQ : 0;
  const int nqs = (p.Nq + C::BQ - 1) / C::BQ;
  const int per_head = nqs > qs0 ? nqs - qs0 : 0;
  const int n_steps = per_head * n_heads;

  // DMA of step t (Q, dO rows and their stats) into ring stage S.
  auto issue = [&]<int S>(int t) {
    const int hl = t / per_head;
    const int qs = qs0 + (t - hl * per_head);
    const int hq = g * p.group + hs + hl * p.hsplit;
    const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
    const int q0 = qs * C::BQ;
    const rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(p.q) + qhead * D, (uint32_t)p.Nq * C::ROWB);
    const rsrc_t ro = make_rsrc(static_cast<const uint16_t*>(p.dout) + qhead * D, (uint32_t)p.Nq * C::ROWB);
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int i = wave * C::DPW + u;
      const bool isd = i >= C::CH;
      const int ci = isd ? i - C::CH : i;
      const int slot = ci * 64 + lane;
      const int row = slot / C::NCH;
      const int c = (slot % C::NCH) ^ swz_kt<D>(row);
      lds_t* dst = (isd ? ost.template operator()<S>() : qst.template operator()<S>()) + ci * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isd ? ro : rq, dst, 16, (q0 + row) * C::ROWB + c * 16,
                                               0, 0, 0);
    }
    if (wave == 0) {
      const rsrc_t rs = make_rsrc(p.stats + qhead, (uint32_t)p.Nq * 8u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, sst.template operator()<S>(), 4, q0 * 8 + lane * 4,
                                               0, 0, 0);
    }
  };
  // End of a step: the next step's transfers (the last ones this wave
  // issued) have landed, and every wave is done with the current stage.
  auto wait_step = [&]() {
    wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (n_steps > 0) issue.template operator()<0>(0);
  wait_vm_lgkm<0>();   // V, K registers (and step 0) complete for this wave
  __builtin_amdgcn_s_barrier();

  const int kbase = l32 * C::ROWB + ((half ^ (swz_kt<D>(l32) & 1)) * 16) + ((swz_kt<D>(l32) >> 1) * 32);
  const int tb0 = tr_base_bwd<D>(lane, 0), tb1 = tr_base_bwd<D>(lane, 1);

  f32x16 adv[D / 32], adk[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    adv[i] = f32x16{};
    adk[i] = f32x16{};
  }

  auto step = [&]<int S>(int t) {
    const bool more = t + 1 < n_steps;
    if (more) issue.template operator()<S ^ 1>(t + 1);
    const int hl = t / per_head;
    const int q0 = (qs0 + (t - hl * per_head)) * C::BQ;
    const lds_t* qs = qst.template operator()<S>();
    const lds_t* os = ost.template operator()<S>();
    const lds_t* ss = sst.template operator()<S>();
    int kb = kbase, vb = wave * 32 * C::ROWB + kbase, t0 = tb0, t1 = tb1;
    asm volatile("" : "+v"(kb), "+v"(vb), "+v"(t0), "+v"(t1));
    // S = Q K^T and dP = dO V^T: one query per register row, this lane's key.
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) {
      const u32x4 a = *(const u32x4 __attribute__((address_space(3)))*)(qs + (kb ^ (cd * 32)));
      sc = M::mma(a, kreg[cd], sc);
    }
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) {
      const u32x4 a = *(const u32x4 __attribute__((address_space(3)))*)(os + (kb ^ (cd * 32)));
      const u32x4 bv = *(const u32x4 __attribute__((address_space(3)))*)((const lds_t*)vall + (vb ^ (cd * 32)));
      dp = M::mma(a, bv, dp);
    }
    // P and dS; register e holds query q0 + (e/4)*8 + half*4 + e%4.
    u32x4 pk[2], dk2[2];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 s01 = *(const f32x4 __attribute__((address_space(3)))*)(ss + (g4 * 8 + half * 4) * 8);
      const f32x4 s23 = *(const f32x4 __attribute__((address_space(3)))*)(ss + (g4 * 8 + half * 4) * 8 + 16);
      const float l2v[4] = {s01[0], s01[2], s23[0], s23[2]};
      const float dv4[4] = {s01[1], s01[3], s23[1], s23[3]};
      float pe[4], de[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = g4 * 4 + j;
        float x = fast_exp2(fmaf(sc[e], p.sl2, -l2v[j]));
        if (CAUSAL && key > q0 + g4 * 8 + half * 4 + j) x = 0.f;
        pe[j] = x;
        de[j] = x * (dp[e] - dv4[j]);
      }
      const int cc = g4 >> 1, w0 = (g4 & 1) * 2;
      pk[cc][w0] = M::pack(pe[0], pe[1]);
      pk[cc][w0 + 1] = M::pack(pe[2], pe[3]);
      dk2[cc][w0] = M::pack(de[0], de[1]);
      dk2[cc][w0 + 1] = M::pack(de[2], de[3]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (transposed operand reads).
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int off = cc * 16 * C::ROWB;
        const s16x4 olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(os + (t0 ^ (db * 64)) + off));
        const s16x4 ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(os + (t1 ^ (db * 64)) + off));
        const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(qs + (t0 ^ (db * 64)) + off));
        const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(qs + (t1 ^ (db * 64)) + off));
        const u32x2 a0 = __builtin_bit_cast(u32x2, olo), a1 = __builtin_bit_cast(u32x2, ohi);
        const u32x2 b0 = __builtin_bit_cast(u32x2, qlo), b1 = __builtin_bit_cast(u32x2, qhi);
        adv[db] = M::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, pk[cc], adv[db]);
        adk[db] = M::mma(u32x4{b0[0], b0[1], b1[0], b1[1]}, dk2[cc], adk[db]);
      }
    }
    wait_step();
  };
  int t = 0;
  for (; t + 1 < n_steps; t += 2) {
    step.template operator()<0>(t);
    step.template operator()<1>(t + 1);
  }
  if (t < n_steps) step.template operator()<0>(t);

  if (p.hsplit > 1) {
    // Partial sums of this head share, fp32, for the reduction pass.
    if (key < p.Nkv) {
      const size_t nkvd = (size_t)p.B * p.Hkv * p.Nkv * D;
      float* pk_ = p.part + (size_t)hs * 2 * nkvd + (kvhead + key) * D;
      float* pv_ = pk_ + nkvd;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int dim = db * 32 + g4 * 8 + half * 4;
          *reinterpret_cast<f32x4*>(pk_ + dim) =
              f32x4{adk[db][4 * g4], adk[db][4 * g4 + 1], adk[db][4 * g4 + 2], adk[db][4 * g4 + 3]} * p.scale;
          *reinterpret_cast<f32x4*>(pv_ + dim) =
              f32x4{adv[db][4 * g4], adv[db][4 * g4 + 1], adv[db][4 * g4 + 2], adv[db][4 * g4 + 3]};
        }
      }
    }
    return;
  }
  // dV and dK rows of this lane's key: 4 consecutive dims per store.
  const rsrc_t rdk = make_rsrc(static_cast<uint16_t*>(p.dk) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rdv = make_rsrc(static_cast<uint16_t*>(p.dv) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int off = (key * D + db * 32 + g4 * 8 + half * 4) * 2;
      u32x2 w;
      w[0] = M::pack(adv[db][4 * g4], adv[db][4 * g4 + 1]);
      w[1] = M::pack(adv[db][4 * g4 + 2], adv[db][4 * g4 + 3]);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, w), rdv, off, 0, 0);
      w[0] = M::pack(adk[db][4 * g4] * p.scale, adk[db][4 * g4 + 1] * p.scale);
      w[1] = M::pack(adk[db][4 * g4 + 2] * p.scale, adk[db][4 * g4 + 3] * p.scale);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, w), rdk, off, 0, 0);
    }
  }
}

// Causal backward grids are persistent, as the causal forward's: min(items,
// CUs) workgroups, one per CU, take the ranks bid, 2G - 1 - bid, 2G + bid,
// 4G - 1 - bid, ... of the longest-first item order (G workgroups), so that
// no workgroup waits for the dispatcher between short items.  Each item ends
// with no transfer in flight; the barrier keeps the next item's transfers
// out of the LDS until every wave has finished reading it.
template <typename F>
__device__ __forceinline__ void persistent_items(int n_items, F&& body) {
  const int G = (int)gridDim.x, bid = (int)blockIdx.x;
  for (int j = 0;; ++j) {
    const int r = (j & 1) ? (j + 1) * G - 1 - bid : j * G + bid;
    if (r >= n_items) break;   // every later rank of this workgroup is larger
    if (j) __syncthreads();
    body(r);
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(CfgBwdKV<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv(BwdParams p) {
  if constexpr (CAUSAL)
    persistent_items(p.items, [&](int r) { attn_bwd_dkdv_body<T, D, true>(p, r, p.items); });
  else
    attn_bwd_dkdv_body<T, D, false>(p, (int)blockIdx.x, (int)gridDim.x);
}

// dK, dV = sum over the head shares of their fp32 partials, in share order
// (deterministic), rounded once.  4 elements per thread.
template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_reduce(const float* __restrict__ part, T* __restrict__ dk,
                                                        T* __restrict__ dv, long long n4, int hsplit) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;   // index of 4 elements
  if (i >= 2 * n4) return;
  const bool isv = i >= n4;
  const long long j = isv ? i - n4 : i;
  const size_t stride = (size_t)2 * n4 * 4;                          // floats per head share
  const float* src = part + (isv ? (size_t)n4 * 4 : 0) + (size_t)j * 4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int h = 1; h < hsplit; ++h) acc += *reinterpret_cast<const f32x4*>(src + h * stride);
  T o4[4] = {(T)acc[0], (T)acc[1], (T)acc[2], (T)acc[3]};
  *reinterpret_cast<u32x2*>((isv ? dv : dk) + j * 4) = __builtin_bit_cast(u32x2, o4);
}

template <int D>
struct CfgBwdQ {
  static constexpr int NW = 8;                  // waves; 32 query rows each
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;            // query rows per workgroup
  static constexpr int BC = 32;                 // keys per tile
  static constexpr int ROWB = D * 2;
  static constexpr int NCH = D / 8;
  static constexpr int TILEB = BC * ROWB;
  static constexpr int CH = TILEB / 1024;       // chunks per K (or V) tile
  static constexpr int DPW = 2 * CH / NW;
  static_assert(DPW >= 1 && DPW * NW == 2 * CH, "DMA split");
};

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dq_body(const BwdParams& p, int item, int n_items) {
  using C = CfgBwdQ<D>;
  using M = Mma16<T>;
  __shared__ __attribute__((aligned(1024))) unsigned char k0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k2s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char k3s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v2s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) unsigned char v3s[C::TILEB];
  auto kst = [&]<int S>() -> lds_t* {
    if constexpr ((S & 3) == 0) return (lds_t*)k0s;
    else if constexpr ((S & 3) == 1) return (lds_t*)k1s;
    else if constexpr ((S & 3) == 2) return (lds_t*)k2s;
    else return (lds_t*)k3s;
  };
  auto vst = [&]<int S>() -> lds_t* {
    if constexpr ((S & 3) == 0) return (lds_t*)v0s;
    else if constexpr ((S & 3) == 1) return (lds_t*)v1s;
    else if constexpr ((S & 3) == 2) return (lds_t*)v2s;
    else return (lds_t*)v3s;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Work item: (b, query head, query tile).  Non-causal: query tiles fastest.
  // Causal: the last query tiles see the most keys; they are listed first,
  // (b, head) fastest.
  const int n_bh = n_items / p.n_tiles;
  const int xl = xcd_local(item, n_items);
  const int qt = CAUSAL ? p.n_tiles - 1 - item / n_bh : xl % p.n_tiles;
  const int bh = CAUSAL ? item % n_bh : xl / p.n_tiles;
  const int hq = bh % p.Hq;
  const int b = bh / p.Hq;
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;

  const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
  const size_t kvhead = (size_t)(b * p.Hkv + hkv) * p.Nkv;
  const rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(p.q) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const rsrc_t rdo = make_rsrc(static_cast<const uint16_t*>(p.dout) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);

  const int kv_end = CAUSAL ? min(p.Nkv, q0 + C::BR) : p.Nkv;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;

  auto issue = [&]<int S>(int t) {
    const int kv0 = t * C::BC;
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int i = wave * C::DPW + u;
      const bool isv = i >= C::CH;
      const int ci = isv ? i - C::CH : i;
      const int slot = ci * 64 + lane;
      const int row = slot / C::NCH;
      const int c = (slot % C::NCH) ^ swz_kt<D>(row);
      lds_t* dst = (isv ? vst.template operator()<S>() : kst.template operator()<S>()) + ci * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, dst, 16, (kv0 + row) * C::ROWB + c * 16,
                                               0, 0, 0);
    }
  };
  // Tile t landed for every wave; tile t+3 goes into the stage tile t-1 held.
  auto advance = [&]<int S>(int t) {
    const int ahead = min(n_tiles - 1 - t, 2);   // groups issued after tile t
    if (ahead >= 2) wait_vm_lgkm<2 * C::DPW>();
    else if (ahead == 1) wait_vm_lgkm<C::DPW>();
    else wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 3 < n_tiles) issue.template operator()<S>(t + 3);
  };

  if (n_tiles > 0) issue.template operator()<0>(0);
  if (n_tiles > 1) issue.template operator()<1>(1);
  if (n_tiles > 2) issue.template operator()<2>(2);

  // Q^T and dO^T operands of the wave's 32 rows, and their statistics.
  u32x4 qreg[D / 16], oreg[D / 16];
#pragma unroll
  for (int cd = 0; cd < D / 16; ++cd) {
    const int off = (myq * D + cd * 16 + half * 8) * 2;
    qreg[cd] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    oreg[cd] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, off, 0, 0));
  }
  const float2 st = myq < p.Nq ? p.stats[qhead + myq] : make_float2(0.f, 0.f);
  const float l2v = st.x, dvv = st.y;

  const int kbase = l32 * C::ROWB + ((half ^ (swz_kt<D>(l32) & 1)) * 16) + ((swz_kt<D>(l32) >> 1) * 32);
  const int tb0 = tr_base_bwd<D>(lane, 0), tb1 = tr_base_bwd<D>(lane, 1);

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  auto step = [&]<int R>(int t) {
    advance.template operator()<(R + 3) & 3>(t);
    const lds_t* ks = kst.template operator()<R>();
    const lds_t* vs = vst.template operator()<R>();
    int kb = kbase, t0 = tb0, t1 = tb1;
    asm volatile("" : "+v"(kb), "+v"(t0), "+v"(t1));
    // S^T = K Q^T and dP^T = V dO^T: this lane's query, keys in registers.
    f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) {
      const u32x4 a = *(const u32x4 __attribute__((address_space(3)))*)(ks + (kb ^ (cd * 32)));
      const u32x4 av = *(const u32x4 __attribute__((address_space(3)))*)(vs + (kb ^ (cd * 32)));
      sc = M::mma(a, qreg[cd], sc);
      dp = M::mma(av, oreg[cd], dp);
    }
    const int kv0 = t * C::BC;
    u32x4 dsk[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float d2[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = cc * 8 + 2 * w + j;
          float x = fast_exp2(fmaf(sc[e], p.sl2, -l2v));
          const int kk = kv0 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (CAUSAL && kk > myq) x = 0.f;
          d2[j] = x * (dp[e] - dvv);
        }
        dsk[cc][w] = M::pack(d2[0], d2[1]);
      }
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int off = cc * 16 * C::ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(ks + (t0 ^ (db * 64)) + off));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(ks + (t1 ^ (db * 64)) + off));
        const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi);
        acc[db] = M::mma(u32x4{a0[0], a0[1], a1[0], a1[1]}, dsk[cc], acc[db]);
      }
    }
  };
  int t = 0;
  for (; t + 4 <= n_tiles; t += 4) {
    step.template operator()<0>(t);
    step.template operator()<1>(t + 1);
    step.template operator()<2>(t + 2);
    step.template operator()<3>(t + 3);
  }
  for (; t < n_tiles; ++t) {
    switch (t & 3) {
      case 0: step.template operator()<0>(t); break;
      case 1: step.template operator()<1>(t); break;
      case 2: step.template operator()<2>(t); break;
      default: step.template operator()<3>(t); break;
    }
  }

  const rsrc_t rdq = make_rsrc(static_cast<uint16_t*>(p.dq) + qhead * D, (uint32_t)p.Nq * C::ROWB);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      u32x2 w;
      w[0] = M::pack(acc[db][4 * g4] * p.scale, acc[db][4 * g4 + 1] * p.scale);
      w[1] = M::pack(acc[db][4 * g4 + 2] * p.scale, acc[db][4 * g4 + 3] * p.scale);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, w), rdq,
                                            (myq * D + db * 32 + g4 * 8 + half * 4) * 2, 0, 0);
    }
  }
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(CfgBwdQ<D>::NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq(BwdParams p) {
  if constexpr (CAUSAL)
    persistent_items(p.items, [&](int r) { attn_bwd_dq_body<T, D, true>(p, r, p.items); });
  else
    attn_bwd_dq_body<T, D, false>(p, (int)blockIdx.x, (int)gridDim.x);
}

// ------------------------------------------------------------- fp32 path

template <int D>
struct CfgF32 {
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int BR = 32 * NW;
  static constexpr int BC = 32;
  static constexpr int KP = D + 4;    // floats; rows shift by 4 banks
  static constexpr int VP = D + 8;    // floats; keys k and k+4 land 32 banks apart
  static constexpr int KTILE = BC * KP;
  static constexpr int VTILE = BC * VP;
  static constexpr int BUF = KTILE + VTILE;
  static constexpr int LDS_BYTES = 2 * BUF * 4;
  static constexpr int LOADS = BC * D / 4 / NT;   // float4 chunks per thread, per tensor
  static_assert(LOADS >= 1 && BC * D / 4 == LOADS * NT, "tile split");
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(CfgF32<D>::NT)
attn_fwd_mfma_f32(Params p) {
  using C = CfgF32<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char fa_smem[];
  float* smem = reinterpret_cast<float*>(fa_smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int b, hq, qt;
  map_block(p, CAUSAL, b, hq, qt);
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + l32;

  const float* Qg = static_cast<const float*>(p.q) + (size_t)(b * p.Hq + hq) * p.Nq * D;
  const float* Kg = static_cast<const float*>(p.k) + (size_t)(b * p.Hkv + hkv) * p.Nkv * D;
  const float* Vg = static_cast<const float*>(p.v) + (size_t)(b * p.Hkv + hkv) * p.Nkv * D;

  // Contraction slot `half` of MFMA step c covers dim half*(D/2) + c, so each
  // lane's dims are contiguous: Q^T operand = Q[myq][half*D/2 .. +D/2).
  float qreg[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; c += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (myq < p.Nq) x = *reinterpret_cast<const f32x4*>(Qg + (size_t)myq * D + half * (D / 2) + c);
    if (p.qmode == 1) x = -x;
    else if (p.qmode == 2) x = f32x4{0.f, 0.f, 0.f, 0.f};
    qreg[c] = x[0];
    qreg[c + 1] = x[1];
    qreg[c + 2] = x[2];
    qreg[c + 3] = x[3];
  }

  const int kv_end = CAUSAL ? min(p.Nkv, q0 + C::BR) : p.Nkv;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  f32x4 kpre[C::LOADS];
  f32x4 vpre[C::LOADS];

  auto load_tile = [&](int j) {
    const int kv0 = j * C::BC;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (kv0 + row < p.Nkv) {
        kx = *reinterpret_cast<const f32x4*>(Kg + (size_t)(kv0 + row) * D + col);
        vx = *reinterpret_cast<const f32x4*>(Vg + (size_t)(kv0 + row) * D + col);
      }
      kpre[i] = kx;
      vpre[i] = vx;
    }
  };
  auto store_tile = [&](int buf) {
    float* Ks = smem + buf * C::BUF;
    float* Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int c = tid + i * C::NT;
      const int row = c / (D / 4);
      const int col = (c % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(Ks + row * C::KP + col) = kpre[i];
      *reinterpret_cast<f32x4*>(Vs + row * C::VP + col) = vpre[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * C::BC;
    if (j + 1 < n_tiles) load_tile(j + 1);
    const float* Ks = smem + (j & 1) * C::BUF;
    const float* Vs = Ks + C::KTILE;
    const bool active = (qw0 < p.Nq) && (!CAUSAL || kv0 <= qw0 + 31);
    if (active) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 2; c += 4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(Ks + l32 * C::KP + half * (D / 2) + c);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], qreg[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], qreg[c + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], qreg[c + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], qreg[c + 3], s, 0, 0, 0);
      }
      const bool need_mask = (kv0 + C::BC > p.Nkv) || (CAUSAL && kv0 + C::BC - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + (r >> 2) * 8 + half * 4 + (r & 3);
          if ((key >= p.Nkv) || (CAUSAL && key > myq)) s[r] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx * p.sl2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(fmaf(s[r], p.sl2, -m_use));
        s[r] = e;
        ls += e;
      }
      l_run = fmaf(l_run, alpha, ls);
      m_run = m_new;
      if (wave_any(alpha != 1.f)) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[i] *= alpha;
      }
      // Register r of S^T holds key (r/4)*8 + half*4 + r%4 for query l32:
      // contraction slot `half` of step r is that key, so the A operand is
      // V[key][d] with d = db*32 + l32 (row-major V, no transpose needed).
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + half * 4 + (r & 3);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const float a = Vs[key * C::VP + db * 32 + l32];
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[r], acc[db], 0, 0, 0);
        }
      }
    }
    if (j + 1 < n_tiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + xor32(l_run);
  if (myq < p.Nq) {
    const float inv = 1.f / l_tot;
    float* Og = static_cast<float*>(p.o) + ((size_t)(b * p.Hq + hq) * p.Nq + myq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                   acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(Og + db * 32 + g * 8 + half * 4) = w;
      }
    }
    if (half == 0) p.lse[(size_t)(b * p.Hq + hq) * p.Nq + myq] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

// ------------------------------------------------------------ host side

thread_local char g_hip_error[256] = "";

struct Geometry {
  int rows_per_block;
  int keys_per_tile;
  int threads;
  int lds_bytes;
};

Geometry geometry_for(int d, int dtype) {
  if (dtype == FA_F32) {
    if (d == 64) return {CfgF32<64>::BR, CfgF32<64>::BC, CfgF32<64>::NT, CfgF32<64>::LDS_BYTES};
    return {CfgF32<128>::BR, CfgF32<128>::BC, CfgF32<128>::NT, CfgF32<128>::LDS_BYTES};
  }
  if (d == 64) return {CfgW64<64>::BR, CfgW64<64>::BC, CfgW64<64>::NT, CfgW64<64>::LDS_BYTES};
  return {CfgW64<128>::BR, CfgW64<128>::BC, CfgW64<128>::NT, CfgW64<128>::LDS_BYTES};
}

size_t elem_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

int check_dims(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int dtype, long long* blocks) {
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || N_q < 1 || N_kv < 1) return FA_ERR_BAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  const Geometry g = geometry_for(d, dtype);
  const long long tiles = ((long long)N_q + g.rows_per_block - 1) / g.rows_per_block;
  const long long nb = (long long)B * Hq * tiles;
  if (nb > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  // Head offsets are 64-bit, but (b * H + h), row indices and the byte
  // offsets inside one head (buffer descriptors, 32-bit) are not.
  if ((long long)B * Hq > 0x7fffffffLL || (long long)B * Hkv > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  const long long nmax = (N_q > N_kv ? N_q : N_kv) + 256LL;
  if (nmax * d * (long long)elem_size(dtype) > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  if (blocks) *blocks = nb;
  return FA_OK;
}

bool overlaps(uintptr_t a, size_t na, uintptr_t b, size_t nb) {
  return a < b + nb && b < a + na;
}

template <typename Kernel>
int launch(Kernel kern, int lds_bytes, const Params& p, long long blocks, int threads,
           hipStream_t stream) {
  (void)hipGetLastError();   // clear a stale error so the check below is ours
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads), lds_bytes, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

template <typename Kernel>
int set_lds_limit(Kernel kern, int lds_bytes) {
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

template <int D, bool CAUSAL>
int run32(const Params& p, long long blocks, hipStream_t stream) {
  using C = CfgF32<D>;
  static const int attr = set_lds_limit(attn_fwd_mfma_f32<D, CAUSAL>, C::LDS_BYTES);
  if (attr != FA_OK) return attr;
  return launch(attn_fwd_mfma_f32<D, CAUSAL>, C::LDS_BYTES, p, blocks, C::NT, stream);
}

// Compute units of the device `stream` runs on (cached per device).
int cu_count(hipStream_t stream, int* out) {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= 64)) e = hipErrorInvalidDevice;
  if (e == hipSuccess) {
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) e = hipDeviceGetAttribute(&cached[dev], hipDeviceAttributeMultiprocessorCount, dev);
    *out = cached[dev];
  }
  if (e != hipSuccess || *out < 1) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

template <typename T, bool CAUSAL, int D>
int run_w64(const Params& p, long long blocks, hipStream_t stream) {
  if constexpr (CAUSAL) {   // persistent grid: one workgroup per CU at most
    int cus = 0;
    const int st = cu_count(stream, &cus);
    if (st != FA_OK) return st;
    blocks = blocks < cus ? blocks : cus;
  }
  return launch(attn_fwd_w64<T, CAUSAL, D>, 0, p, blocks, CfgW64<D>::NT, stream);
}

template <typename T>
int dispatch16(const Params& p, int d, bool causal, long long blocks, hipStream_t s) {
  if (d == 64) return causal ? run_w64<T, true, 64>(p, blocks, s) : run_w64<T, false, 64>(p, blocks, s);
  return causal ? run_w64<T, true, 128>(p, blocks, s) : run_w64<T, false, 128>(p, blocks, s);
}

template <int D, bool CAUSAL>
int run8(const Params& p, long long blocks, hipStream_t stream) {
  if constexpr (D == 128) {   // the 64-row body; causal grids persistent as in run_w64
    if constexpr (CAUSAL) {
      int cus = 0;
      const int st = cu_count(stream, &cus);
      if (st != FA_OK) return st;
      blocks = blocks < cus ? blocks : cus;
    }
    return launch(attn_fwd_w64_e4m3<CAUSAL>, 0, p, blocks, CfgW64E::NT, stream);
  }
  return launch(attn_fwd_e4m3<D, CAUSAL>, 0, p, blocks, Cfg8<D>::NT, stream);
}

// Host checks of the FP8 entry point (dimensions as for the 16-bit path with
// 2-byte output elements; the 1-byte inputs are covered by the same limits).
int check_fp8_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   int B, int Hq, int Hkv, int N_q, int N_kv, int d, float scale, float dsq,
                   float dsk, float dsv, long long* blocks) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  const int st = check_dims(B, Hq, Hkv, N_q, N_kv, d, FA_BF16, blocks);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  if (!(isfinite(dsq) && dsq > 0.f) || !(isfinite(dsk) && dsk > 0.f) || !(isfinite(dsv) && dsv > 0.f))
    return FA_ERR_SCALE;
  const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v, po = (uintptr_t)o,
                  pl = (uintptr_t)lse;
  if (((pq | pk | pv | po) & 15u) != 0 || (pl & 3u) != 0) return FA_ERR_ALIGN;
  const size_t nq = (size_t)B * Hq * N_q * d;
  const size_t nkv = (size_t)B * Hkv * N_kv * d;
  const size_t no = nq * 2;
  const size_t nl = (size_t)B * Hq * N_q * sizeof(float);
  if (overlaps(po, no, pq, nq) || overlaps(po, no, pk, nkv) || overlaps(po, no, pv, nkv) ||
      overlaps(pl, nl, pq, nq) || overlaps(pl, nl, pk, nkv) || overlaps(pl, nl, pv, nkv) ||
      overlaps(po, no, pl, nl))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// Split-KV geometry for valid dimensions (d, dtype already checked).
struct SplitGeometry {
  int R, nrb, n_tiles;   // packed rows per kv head, row blocks, 32-key tiles of N_kv
};

SplitGeometry split_geometry(int Hq, int Hkv, int N_q, int N_kv) {
  SplitGeometry g;
  g.R = (Hq / Hkv) * N_q;
  g.nrb = (g.R + 31) / 32;
  g.n_tiles = (N_kv + 31) / 32;
  return g;
}

int check_split_dims(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int dtype, int num_splits) {
  if (dtype == FA_F32) return FA_ERR_DTYPE;
  const int st = check_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, nullptr);
  if (st != FA_OK) return st;
  if ((long long)(Hq / Hkv) * N_q > 0x7fffffffLL - 32) return FA_ERR_BAD_DIM;
  const SplitGeometry g = split_geometry(Hq, Hkv, N_q, N_kv);
  if (num_splits < 1 || num_splits > g.n_tiles || num_splits > FA_SPLITKV_MAX_SPLITS)
    return FA_ERR_BAD_DIM;
  const long long items = (long long)B * Hkv * g.nrb * num_splits;
  if ((items + 7) / 8 > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  if ((long long)B * Hq * N_q > 0x7fffffffLL) return FA_ERR_BAD_DIM;   // one combine block per row
  return FA_OK;
}

template <typename T, int D, bool CAUSAL, bool PAGED = false>
int run_split(const SplitParams& sp, T* o, float* lse, hipStream_t stream) {
  using C = CfgSplit<D>;
  (void)hipGetLastError();
  const long long blocks = (sp.items + C::NW - 1) / C::NW;
  hipLaunchKernelGGL((attn_splitkv_mfma16<T, D, CAUSAL, PAGED>), dim3((unsigned)blocks), dim3(C::NT), 0,
                     stream, sp);
  hipLaunchKernelGGL((attn_splitkv_combine<T, D>), dim3((unsigned)sp.rows), dim3(256), 0, stream,
                     sp.ows, sp.lws, o, lse, sp.rows, sp.S);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

template <typename T, bool PAGED = false>
int dispatch_split(const SplitParams& sp, void* o, float* lse, int d, bool causal, hipStream_t s) {
  T* ot = static_cast<T*>(o);
  if (d == 64)
    return causal ? run_split<T, 64, true, PAGED>(sp, ot, lse, s) : run_split<T, 64, false, PAGED>(sp, ot, lse, s);
  return causal ? run_split<T, 128, true, PAGED>(sp, ot, lse, s) : run_split<T, 128, false, PAGED>(sp, ot, lse, s);
}

// Both launches of the split-KV forward once every argument has been checked;
// `workspace` holds fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits) bytes.
int launch_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int N_q, int N_kv, int d, float scale, int causal, int dtype,
                   int num_splits, void* workspace, void* stream) {
  const SplitGeometry g = split_geometry(Hq, Hkv, N_q, N_kv);
  SplitParams sp;
  sp.q = q;
  sp.k = k;
  sp.v = v;
  sp.rows = (long long)B * Hq * N_q;
  sp.ows = static_cast<float*>(workspace);
  sp.lws = sp.ows + (size_t)num_splits * sp.rows * d;
  sp.B = B;
  sp.Hq = Hq;
  sp.Hkv = Hkv;
  sp.Nq = N_q;
  sp.Nkv = N_kv;
  sp.group = Hq / Hkv;
  sp.R = g.R;
  sp.nrb = g.nrb;
  sp.S = num_splits;
  sp.items = (long long)B * Hkv * g.nrb * num_splits;
  if (scale > 0.f) {
    sp.sl2 = scale * kLog2e;
    sp.qmode = 0;
  } else if (scale < 0.f) {
    sp.sl2 = -scale * kLog2e;
    sp.qmode = 1;
  } else {
    sp.sl2 = 1.f;
    sp.qmode = 2;
  }
  sp.btab = nullptr;
  sp.seqlens = nullptr;
  sp.mbps = sp.lbs = sp.nblocks = 0;
  sp.pool_bytes = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  if (dtype == FA_BF16) return dispatch_split<__bf16>(sp, o, lse, d, c, s);
  return dispatch_split<_Float16>(sp, o, lse, d, c, s);
}

template <typename T, int D, bool CAUSAL>
int run_bwd(BwdParams p, long long rows, hipStream_t stream) {
  (void)hipGetLastError();
  const long long pblocks = (rows * (D / 8) + 255) / 256;
  hipLaunchKernelGGL((attn_bwd_prep<T, D>), dim3((unsigned)pblocks), dim3(256), 0, stream, p, rows);
  // Causal grids: one persistent workgroup per CU at most.
  int cus = 0x7fffffff;
  if (CAUSAL) {
    const int st = cu_count(stream, &cus);
    if (st != FA_OK) return st;
  }
  BwdParams pk = p;
  pk.n_tiles = (p.Nkv + CfgBwdKV<D>::BKV - 1) / CfgBwdKV<D>::BKV;
  pk.items = p.B * p.Hkv * p.hsplit * pk.n_tiles;
  hipLaunchKernelGGL((attn_bwd_dkdv<T, D, CAUSAL>), dim3((unsigned)min(pk.items, cus)),
                     dim3(CfgBwdKV<D>::NT), 0, stream, pk);
  if (p.hsplit > 1) {
    const long long n4 = (long long)p.B * p.Hkv * p.Nkv * D / 4;
    hipLaunchKernelGGL((attn_bwd_reduce<T>), dim3((unsigned)((2 * n4 + 255) / 256)), dim3(256), 0,
                       stream, (const float*)p.part, static_cast<T*>(p.dk), static_cast<T*>(p.dv),
                       n4, p.hsplit);
  }
  BwdParams pq = p;
  pq.n_tiles = (p.Nq + CfgBwdQ<D>::BR - 1) / CfgBwdQ<D>::BR;
  pq.items = p.B * p.Hq * pq.n_tiles;
  hipLaunchKernelGGL((attn_bwd_dq<T, D, CAUSAL>), dim3((unsigned)min(pq.items, cus)),
                     dim3(CfgBwdQ<D>::NT), 0, stream, pq);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

template <typename T>
int dispatch_bwd(const BwdParams& p, long long rows, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? run_bwd<T, 64, true>(p, rows, s) : run_bwd<T, 64, false>(p, rows, s);
  return causal ? run_bwd<T, 128, true>(p, rows, s) : run_bwd<T, 128, false>(p, rows, s);
}

}  // namespace

// Device-resident workspace of the allocation-free split-KV entry point
// (fa_fwd_splitkv_noalloc): one copy per GPU, loaded with the library's code
// object and kept until the process ends.  Host code never uses this name as
// an address: it stands for the array only on the device side.  The device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device
// (scratch_address below), and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, looked up on that device's
// first use (with `dev` made current for the lookup, then restored).
int scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: device %d beyond the %d supported", dev,
             kMaxDevices);
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || ptr == nullptr) {
      snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s) looking up the scratch array",
               hipGetErrorName(e), hipGetErrorString(e));
      return FA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int B, int Hq, int Hkv, int N_q, int N_kv, int d, float scale, int causal,
                  int dtype) {
  (void)causal;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL_PTR;
  const int st = check_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, nullptr);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k, pv = (uintptr_t)v, po = (uintptr_t)o,
                  pl = (uintptr_t)lse;
  if (((pq | pk | pv | po) & 15u) != 0 || (pl & 3u) != 0) return FA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * Hq * N_q * d * es;
  const size_t nkv = (size_t)B * Hkv * N_kv * d * es;
  const size_t nl = (size_t)B * Hq * N_q * sizeof(float);
  if (overlaps(po, nq, pq, nq) || overlaps(po, nq, pk, nkv) || overlaps(po, nq, pv, nkv) ||
      overlaps(pl, nl, pq, nq) || overlaps(pl, nl, pk, nkv) || overlaps(pl, nl, pv, nkv) ||
      overlaps(po, nq, pl, nl))
    return FA_ERR_ALIAS;
  return FA_OK;
}

int fa_launch_info(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int causal, int dtype,
                   int* rows_per_block, int* keys_per_tile, int* threads_per_block,
                   long long* blocks, int* lds_bytes) {
  (void)causal;
  long long nb = 0;
  const int st = check_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, &nb);
  if (st != FA_OK) return st;
  const Geometry g = geometry_for(d, dtype);
  if (rows_per_block) *rows_per_block = g.rows_per_block;
  if (keys_per_tile) *keys_per_tile = g.keys_per_tile;
  if (threads_per_block) *threads_per_block = g.threads;
  if (blocks) *blocks = nb;
  if (lds_bytes) *lds_bytes = g.lds_bytes;
  return FA_OK;
}

int fa_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int N_q, int N_kv, int d, float scale, int causal, int dtype,
                  void* stream) {
  const int st = fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  long long blocks = 0;
  check_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, &blocks);
  const Geometry g = geometry_for(d, dtype);

  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.group = Hq / Hkv;
  p.n_qtiles = (N_q + g.rows_per_block - 1) / g.rows_per_block;
  p.n_heads = B * Hq;
  if (scale > 0.f) {
    p.sl2 = scale * kLog2e;
    p.qmode = 0;
  } else if (scale < 0.f) {
    p.sl2 = -scale * kLog2e;
    p.qmode = 1;
  } else {
    p.sl2 = 1.f;
    p.qmode = 2;
  }
  p.oscale = 1.f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  switch (dtype) {
    case FA_BF16: return dispatch16<__bf16>(p, d, c, blocks, s);
    case FA_F16: return dispatch16<_Float16>(p, d, c, blocks, s);
    default:
      if (d == 64) return c ? run32<64, true>(p, blocks, s) : run32<64, false>(p, blocks, s);
      return c ? run32<128, true>(p, blocks, s) : run32<128, false>(p, blocks, s);
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int N_q, int N_kv, int d, float scale, int causal, int dtype) {
  return fa_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype, nullptr);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N_q, int N_kv, int d, float scale, int causal, float descale_q,
               float descale_k, float descale_v, void* stream) {
  long long blocks = 0;
  const int st = check_fp8_args(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, descale_q,
                                descale_k, descale_v, &blocks);
  if (st != FA_OK) return st;
  Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.group = Hq / Hkv;
  p.n_qtiles = (N_q + Cfg8<128>::BR - 1) / Cfg8<128>::BR;
  p.n_heads = B * Hq;
  // Q's and K's factors scale every score: fold them into the exponent scale.
  const double eff = (double)scale * ((double)descale_q * (double)descale_k);   // exact product
  const float mag = (float)(fabs(eff) * (double)kLog2e);
  if (eff != 0.0 && mag > 0.f) {
    p.sl2 = mag;
    p.qmode = eff > 0.0 ? 0 : 1;
  } else {
    p.sl2 = 1.f;
    p.qmode = 2;
  }
  p.oscale = descale_v;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  if (d == 64) return c ? run8<64, true>(p, blocks, s) : run8<64, false>(p, blocks, s);
  return c ? run8<128, true>(p, blocks, s) : run8<128, false>(p, blocks, s);
}

size_t fa_splitkv_workspace_bytes(int B, int Hq, int N_q, int d, int num_splits) {
  if (B < 1 || Hq < 1 || N_q < 1 || (d != 64 && d != 128) || num_splits < 1 ||
      num_splits > FA_SPLITKV_MAX_SPLITS)
    return 0;
  const unsigned long long rows = (unsigned long long)B * Hq * N_q;
  return (size_t)(rows * (unsigned long long)num_splits * (d + 1) * sizeof(float));
}

int fa_splitkv_default_splits(int B, int Hq, int Hkv, int N_q, int N_kv, int d, int dtype) {
  const int st = check_split_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, 1);
  if (st != FA_OK) return 0;
  const SplitGeometry g = split_geometry(Hq, Hkv, N_q, N_kv);
  // About 2048 waves (two rounds of 4 waves on each of the 256 CUs), and at
  // least 4 tiles (128 keys) per chunk so the merge stays cheap.
  const long long base = (long long)B * Hkv * g.nrb;
  long long s = (2048 + base - 1) / base;
  const long long cap = (g.n_tiles + 3) / 4;
  if (s > cap) s = cap;
  if (s > FA_SPLITKV_MAX_SPLITS) s = FA_SPLITKV_MAX_SPLITS;
  return s < 1 ? 1 : (int)s;
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int N_q, int N_kv, int d, float scale, int causal, int dtype,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return FA_ERR_NULL_PTR;
  int st = fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  st = check_split_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, num_splits);
  if (st != FA_OK) return st;
  const size_t need = fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const uintptr_t pw = (uintptr_t)workspace;
  if ((pw & 15u) != 0) return FA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * Hq * N_q * d * es;
  const size_t nkv = (size_t)B * Hkv * N_kv * d * es;
  const size_t nl = (size_t)B * Hq * N_q * sizeof(float);
  if (overlaps(pw, need, (uintptr_t)q, nq) || overlaps(pw, need, (uintptr_t)k, nkv) ||
      overlaps(pw, need, (uintptr_t)v, nkv) || overlaps(pw, need, (uintptr_t)o, nq) ||
      overlaps(pw, need, (uintptr_t)lse, nl))
    return FA_ERR_ALIAS;

  return launch_splitkv(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype,
                        num_splits, workspace, stream);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int N_q, int N_kv, int d, float scale,
                           int causal, int dtype, int num_splits, void* stream) {
  int st = fa_check_args(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  st = check_split_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, num_splits);
  if (st != FA_OK) return st;
  const size_t need = fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits);
  if (need == 0 || need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  const hipError_t e = hipStreamGetDevice(s, &dev);
  if (e != hipSuccess) {
    snprintf(g_hip_error, sizeof g_hip_error, "HIP error: %s (%s)", hipGetErrorName(e),
             hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != FA_OK) return st;
  return launch_splitkv(q, k, v, o, lse, B, Hq, Hkv, N_q, N_kv, d, scale, causal, dtype,
                        num_splits, ws, stream);
}

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                 const int* seqlens_k, void* o, float* lse, int B, int Hq, int Hkv, int N_q, int d,
                 int num_blocks, int block_size, int max_blocks_per_seq, float scale, int causal,
                 int dtype, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seqlens_k || !o || !lse || !workspace)
    return FA_ERR_NULL_PTR;
  if (dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (B < 1 || Hq < 1 || Hkv < 1 || N_q < 1 || num_blocks < 1 || max_blocks_per_seq < 1)
    return FA_ERR_BAD_DIM;
  if (Hq % Hkv != 0) return FA_ERR_HEAD_GROUP;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (block_size < 16 || block_size > (1 << 16) || (block_size & (block_size - 1)) != 0)
    return FA_ERR_BAD_DIM;
  int lbs = 0;
  while ((1 << lbs) < block_size) ++lbs;
  const long long max_len = (long long)max_blocks_per_seq << lbs;
  if (max_len > 0x7fffffffLL - 64) return FA_ERR_BAD_DIM;
  const size_t es = elem_size(dtype);
  const unsigned long long pool = (unsigned long long)num_blocks * block_size * Hkv * d * es;
  if (pool > 0xffffffffULL - 4096) return FA_ERR_BAD_DIM;   // 32-bit buffer offsets
  if ((long long)B * max_blocks_per_seq > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  int st = check_split_dims(B, Hq, Hkv, N_q, (int)max_len, d, dtype, num_splits);
  if (st != FA_OK) return st;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const size_t need = fa_splitkv_workspace_bytes(B, Hq, N_q, d, num_splits);
  if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  const uintptr_t pq = (uintptr_t)q, pk = (uintptr_t)k_cache, pv = (uintptr_t)v_cache,
                  po = (uintptr_t)o, pl = (uintptr_t)lse, pt = (uintptr_t)block_table,
                  pn = (uintptr_t)seqlens_k, pw = (uintptr_t)workspace;
  if (((pq | pk | pv | po | pw) & 15u) != 0 || ((pl | pt | pn) & 3u) != 0) return FA_ERR_ALIGN;
  const size_t nq = (size_t)B * Hq * N_q * d * es;
  const size_t nl = (size_t)B * Hq * N_q * sizeof(float);
  const size_t nt = (size_t)B * max_blocks_per_seq * sizeof(int);
  const size_t nn = (size_t)B * sizeof(int);
  const uintptr_t outs[3] = {po, pl, pw};
  const size_t outn[3] = {nq, nl, need};
  const uintptr_t ins[5] = {pq, pk, pv, pt, pn};
  const size_t inn[5] = {nq, (size_t)pool, (size_t)pool, nt, nn};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], outn[i], ins[j], inn[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outn[i], outs[j], outn[j])) return FA_ERR_ALIAS;
  }

  const SplitGeometry g = split_geometry(Hq, Hkv, N_q, (int)max_len);
  SplitParams sp;
  sp.q = q;
  sp.k = k_cache;
  sp.v = v_cache;
  sp.rows = (long long)B * Hq * N_q;
  sp.ows = static_cast<float*>(workspace);
  sp.lws = sp.ows + (size_t)num_splits * sp.rows * d;
  sp.B = B;
  sp.Hq = Hq;
  sp.Hkv = Hkv;
  sp.Nq = N_q;
  sp.Nkv = (int)max_len;
  sp.group = Hq / Hkv;
  sp.R = g.R;
  sp.nrb = g.nrb;
  sp.S = num_splits;
  sp.items = (long long)B * Hkv * g.nrb * num_splits;
  if (scale > 0.f) {
    sp.sl2 = scale * kLog2e;
    sp.qmode = 0;
  } else if (scale < 0.f) {
    sp.sl2 = -scale * kLog2e;
    sp.qmode = 1;
  } else {
    sp.sl2 = 1.f;
    sp.qmode = 2;
  }
  sp.btab = block_table;
  sp.seqlens = seqlens_k;
  sp.mbps = max_blocks_per_seq;
  sp.lbs = lbs;
  sp.nblocks = num_blocks;
  sp.pool_bytes = (uint32_t)pool;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  if (dtype == FA_BF16) return dispatch_split<__bf16, true>(sp, o, lse, d, c, s);
  return dispatch_split<_Float16, true>(sp, o, lse, d, c, s);
}

}  // extern "C"

namespace {
// Head shares of the dK/dV pass: enough workgroups for about eight per CU,
// never more shares than query heads per key/value head.
int bwd_hsplit(int B, int Hq, int Hkv, int N_kv) {
  const long long base = (long long)B * Hkv * ((N_kv + 255) / 256);
  long long hs = (2048 + base - 1) / base;
  const int group = Hq / Hkv;
  if (hs > group) hs = group;
  return hs < 1 ? 1 : (int)hs;
}
}  // namespace

extern "C" {

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int N_q, int N_kv, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N_q < 1 || N_kv < 1 || Hq % Hkv != 0 || (d != 64 && d != 128))
    return 0;
  const unsigned long long stats = (unsigned long long)B * Hq * N_q * 8ull;
  const int hs = bwd_hsplit(B, Hq, Hkv, N_kv);
  const unsigned long long part =
      hs > 1 ? (unsigned long long)hs * 2ull * B * Hkv * N_kv * d * 4ull : 0ull;
  return (size_t)(((stats + 255) / 256) * 256 + part);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N_q,
           int N_kv, int d, float scale, int causal, int dtype, void* workspace,
           size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return FA_ERR_NULL_PTR;
  if (dtype == FA_F32) return FA_ERR_DTYPE;
  int st = check_dims(B, Hq, Hkv, N_q, N_kv, d, dtype, nullptr);
  if (st != FA_OK) return st;
  const long long kvtiles = ((long long)N_kv + 255) / 256;
  if ((long long)B * Hkv * kvtiles > 0x7fffffffLL) return FA_ERR_BAD_DIM;
  if (!isfinite(scale)) return FA_ERR_SCALE;
  const uintptr_t in[6] = {(uintptr_t)q, (uintptr_t)k, (uintptr_t)v, (uintptr_t)o, (uintptr_t)lse,
                           (uintptr_t)dout};
  const uintptr_t out[4] = {(uintptr_t)dq, (uintptr_t)dk, (uintptr_t)dv, (uintptr_t)workspace};
  if (((in[0] | in[1] | in[2] | in[3] | in[5] | out[0] | out[1] | out[2] | out[3]) & 15u) != 0 ||
      (in[4] & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t es = elem_size(dtype);
  const size_t nq = (size_t)B * Hq * N_q * d * es;
  const size_t nkv = (size_t)B * Hkv * N_kv * d * es;
  const size_t nl = (size_t)B * Hq * N_q * sizeof(float);
  const size_t nws = fa_bwd_workspace_bytes(B, Hq, Hkv, N_q, N_kv, d);
  if (workspace_bytes < nws) return FA_ERR_WORKSPACE;
  const size_t in_n[6] = {nq, nkv, nkv, nq, nl, nq};
  const size_t out_n[4] = {nq, nkv, nkv, nws};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], out_n[i], in[j], in_n[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out_n[i], out[j], out_n[j])) return FA_ERR_ALIAS;
  }
  BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = static_cast<float2*>(workspace);
  p.hsplit = bwd_hsplit(B, Hq, Hkv, N_kv);
  p.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    (((size_t)B * Hq * N_q * 8 + 255) / 256) * 256);
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = N_q;
  p.Nkv = N_kv;
  p.group = Hq / Hkv;
  p.scale = scale;
  p.sl2 = scale * kLog2e;
  p.n_tiles = 0;
  p.items = 0;
  const long long rows = (long long)B * Hq * N_q;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16) return dispatch_bwd<__bf16>(p, rows, d, causal != 0, s);
  return dispatch_bwd<_Float16>(p, rows, d, causal != 0, s);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA_ERR_BAD_DIM: return "a dimension is < 1 or the launch grid would be too large";
    case FA_ERR_HEAD_GROUP: return "Hq is not a multiple of Hkv";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_F32, FA_F16 or FA_BF16";
    case FA_ERR_SCALE: return "scale must be finite";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "o, lse or the workspace overlaps an input or each other";
    case FA_ERR_WORKSPACE:
      return "workspace smaller than needed (or, for the allocation-free entry point, more than "
             "FA_NOALLOC_SCRATCH_BYTES needed)";
    case FA_ERR_HIP: return g_hip_error[0] ? g_hip_error : "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
