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

// ----------------------------------------------- 16-bit (bf16 / f16) path
//
// Workgroup: 8 waves x 32 query rows = 256 rows.  K/V tiles of 64 keys move
// global -> LDS by buffer DMA (buffer_load ... lds, 16 B per lane, no VGPR
// staging; rows past N_kv come back as zeros) into a 4-stage ring, issued two
// tiles ahead.  K is stored row-major with an XOR swizzle of its 16-byte
// chunks (conflict-free 16-byte operand reads); V is stored row-major too,
// with its own swizzle, and read transposed by ds_read_b64_tr_b16, which
// hands each lane four keys of one head-dimension column: the V^T operand of
// the P*V product without any transpose pass.
//
// Main loop (tiles that need no mask), software-pipelined per wave:
//   phase A: MFMA S(j+1) = K(j+1) Q^T   ||  VALU exp(S(j)) -> P(j), row sums
//   phase B: MFMA O += V(j) P(j)        ||  VALU row max of S(j+1), new reference
// Diagonal (causal) and ragged-tail tiles run afterwards through a plain,
// masked, non-pipelined step.
//
// The exponent reference is lazy: it moves to the new running max only when
// that max exceeds it by more than 2^8 (then O and the sum are rescaled by
// exp2(m_old - m_new)).  Otherwise probabilities are taken against the older,
// smaller reference and stay below 2^8.  O / l and lse = ref + log2(l) are
// the same whatever reference is used, so the result stays exact; only the
// rescale work is skipped.

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
};

template <int D>
struct Cfg16 {
  static constexpr int QH = 1;                  // 32-row query halves per wave
  static constexpr int NW = 8;                  // waves per workgroup
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int BR = 32 * QH * NW;       // query rows per workgroup
  static constexpr int BC = 64;                 // keys per K/V tile
  static constexpr int KT = BC / 32;            // 32-key blocks per tile
  static constexpr int WAVES_PER_EU = QH == 1 ? 2 : 1;
  static constexpr int STAGES = 4;              // LDS ring depth (tiles)
  static constexpr int ROWB = D * 2;            // bytes per K/V row
  static constexpr int NCH = D / 8;             // 16-byte chunks per row
  static constexpr int TILEB = BC * ROWB;       // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;      // K tile then V tile
  static constexpr int LDS_BYTES = STAGES * STAGEB;
  static constexpr int CHUNKS = STAGEB / 1024;  // 1 KiB DMA instructions per tile
  static constexpr int DPW = CHUNKS / NW;       // ... per wave
  static_assert(DPW * NW == CHUNKS && DPW >= 1, "DMA split");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
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

// Body of the 16-bit kernel.  It lives in a device function because the
// host compilation pass does not emit launch stubs for kernel templates whose
// own body holds template lambdas.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_mfma16_body(const Params& p) {
  using C = Cfg16<D>;
  constexpr int KT = C::KT;
  constexpr int QH = C::QH;
  using M = Mma16<T>;
  // One LDS object per ring stage and operand: with compile-time stage
  // indices the compiler can tell a read of one stage from a DMA into another
  // and does not stall the read on the unrelated transfer; the K ring fills
  // the first 64 KiB so every K stage offset fits a ds_read immediate.
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int b, hq, qt;
  map_block(p, CAUSAL, b, hq, qt);
  const int hkv = hq / p.group;
  const int q0 = qt * C::BR;
  const int qw0 = q0 + wave * 32 * QH;   // first query row of this wave
  // Query half h of the wave holds rows qw0 + 32h .. +31; lane l32 of it
  // holds row qw0 + 32h + l32 (its O column and its row statistics).

  const size_t qhead = (size_t)(b * p.Hq + hq) * p.Nq;
  const size_t kvhead = (size_t)(b * p.Hkv + hkv) * p.Nkv;
  const rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(p.q) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(p.k) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);
  const rsrc_t rv = make_rsrc(static_cast<const uint16_t*>(p.v) + kvhead * D, (uint32_t)p.Nkv * C::ROWB);

  const int kv_end = CAUSAL ? min(p.Nkv, q0 + C::BR) : p.Nkv;
  const int n_tiles = (kv_end + C::BC - 1) / C::BC;
  // Tiles whose every key is allowed for every row of the workgroup.
  const int n_main = CAUSAL ? min((q0 + 1) / C::BC, p.Nkv / C::BC) : p.Nkv / C::BC;

  // DMA of tile t into ring stage S (= t mod 4).
  auto issue = [&]<int S>(int t) {
    const int kv0 = t * C::BC;
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int i = wave * C::DPW + u;            // 1 KiB chunk of the stage (wave-uniform)
      const bool isv = i >= C::CHUNKS / 2;
      const int ci = isv ? i - C::CHUNKS / 2 : i;
      const int slot = ci * 64 + lane;            // 16-byte slot within the tile
      const int row = slot / C::NCH;
      const int c = (slot % C::NCH) ^ (isv ? swz_v<D>(row) : swz_k<D>(row));
      lds_t* dst = (isv ? vst.template operator()<S>() : kst.template operator()<S>()) + ci * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isv ? rv : rk, (lds_t*)dst, 16,
                                               (kv0 + row) * C::ROWB + c * 16, 0, 0, 0);
    }
  };

  // Tile t has landed in LDS for every wave; tile t+2 (ring stage S) is issued.
  auto advance = [&]<int S>(int t) {
    if (t + 1 < n_tiles) wait_vm_lgkm<C::DPW>();
    else wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 2 < n_tiles) issue.template operator()<S>(t + 2);
  };

  issue.template operator()<0>(0);
  if (n_tiles > 1) issue.template operator()<1>(1);

  // Q^T operand, held for the whole loop: lane (l32, half) has row myq, dims
  // cd*16 + half*8 .. +7.  Rows past N_q read as zeros.  qmode 1 flips both
  // halves' sign bits (exact negation), qmode 2 zeroes Q.
  const uint32_t qxor = p.qmode == 1 ? 0x80008000u : 0u;
  const uint32_t qand = p.qmode == 2 ? 0u : 0xffffffffu;
  u32x4 qreg[QH][D / 16];
#pragma unroll
  for (int h = 0; h < QH; ++h) {
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) {
      const int row = qw0 + 32 * h + l32;
      const u32x4 x = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (row * D + cd * 16 + half * 8) * 2, 0, 0));
      qreg[h][cd] = (x ^ qxor) & qand;
    }
  }

  // Per-lane LDS byte offsets of the operand reads.  The swizzles have a
  // period of 16 rows and act on chunk-index bits that a loop index only
  // XORs, so one base per operand suffices:
  //   K, dims cd*16.. of row l32 (+32 kt):   kbase ^ (cd * 32)   (+ kt * 32 rows)
  //   V^T, columns db*32.., keys as above:   vbase ^ (db * 64)   (+ row offsets)
  const int kbase = l32 * C::ROWB + ((half ^ (swz_k<D>(l32) & 1)) * 16) + ((swz_k<D>(l32) >> 1) * 32);
  const int g16 = lane >> 4, s16 = lane & 15;
  const int vrow = (g16 >> 1) * 4 + (s16 >> 2);
  const int vbase = vrow * C::ROWB + (swz_v<D>(vrow) >> 2) * 64 + (g16 & 1) * 32 +
                    ((s16 & 3) >> 1) * 16 + (s16 & 1) * 8;

  f32x16 acc[QH][D / 32];
#pragma unroll
  for (int h = 0; h < QH; ++h)
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[h][i] = f32x16{};
  float m_run[QH];   // exponent reference (log2 units), shared by both half-waves
  float l_run[QH];   // this lane's part of the row sum, against m_run
#pragma unroll
  for (int h = 0; h < QH; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
  }

  // The lane bases pass through an empty asm in every call so that the
  // compiler recomputes the few XORs per tile instead of hoisting one address
  // register per (stage, chunk) pair out of the loop.
  auto compute_s = [&](const lds_t* st, f32x16 (&s)[QH][KT]) {
    int kb = kbase;
    asm volatile("" : "+v"(kb));
#pragma unroll
    for (int h = 0; h < QH; ++h)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[h][kt] = f32x16{};
#pragma unroll
    for (int cd = 0; cd < D / 16; ++cd) {
      const lds_t* a = st + (kb ^ (cd * 32));
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const u32x4 x = *(const u32x4 __attribute__((address_space(3)))*)(a + kt * 32 * C::ROWB);
#pragma unroll
        for (int h = 0; h < QH; ++h) s[h][kt] = M::mma(x, qreg[h][cd], s[h][kt]);
      }
    }
  };

  auto compute_pv = [&](const lds_t* st, const u32x4 (&pk)[QH][KT][2]) {
    int vb = vbase;
    asm volatile("" : "+v"(vb));
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const lds_t* a0 = st + (vb ^ (db * 64)) + (kt * 32 + cc * 16) * C::ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)a0);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(a0 + 8 * C::ROWB));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 x = {l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
          for (int h = 0; h < QH; ++h) acc[h][db] = M::mma(x, pk[h][kt][cc], acc[h][db]);
        }
      }
    }
  };

  // New exponent reference of query half h from a tile of raw scores;
  // returns the factor that moves earlier sums to it (1 when the reference
  // stays, 0 the first time).
  auto new_reference = [&](const f32x16 (&s)[KT], int h) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = pair_max(mx);
    const float mc = mx * p.sl2;
    const float m_new = (mc > m_run[h] + kLazy) ? mc : m_run[h];
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[h] - m_new);
    m_run[h] = m_new;
    return alpha;
  };

  auto rescale = [&](const float (&alpha)[QH]) {
    bool any = false;
#pragma unroll
    for (int h = 0; h < QH; ++h) {
      l_run[h] *= alpha[h];
      any = any || (alpha[h] != 1.f);
    }
    if (wave_any(any)) {
#pragma unroll
      for (int h = 0; h < QH; ++h)
#pragma unroll
        for (int i = 0; i < D / 32; ++i) acc[h][i] *= alpha[h];
    }
  };

  // P = exp2(s * sl2 - ref), rounded to T and packed as the B operand of P*V;
  // the row sum accumulates the rounded values in fp32.
  auto exponentiate = [&](const f32x16 (&s)[KT], u32x4 (&pk)[KT][2], int h) {
    const float mu = (m_run[h] == -INFINITY) ? 0.f : m_run[h];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float e0 = fast_exp2(fmaf(s[kt][cc * 8 + 2 * w], p.sl2, -mu));
          const float e1 = fast_exp2(fmaf(s[kt][cc * 8 + 2 * w + 1], p.sl2, -mu));
          const uint32_t pr = M::pack(e0, e1);
          pk[kt][cc][w] = pr;
          if (w & 1) ls1 = M::sum2(pr, ls1);
          else ls0 = M::sum2(pr, ls0);
        }
      }
    }
    l_run[h] += ls0 + ls1;
  };

  f32x16 s_cur[QH][KT];
  u32x4 pk[QH][KT][2];

  // Steady iteration j (j % 4 == R): tile j+1 is unmasked too.
  auto steady = [&]<int R>(int j) {
    advance.template operator()<(R + 3) & 3>(j + 1);
    f32x16 s_next[QH][KT];
#pragma unroll
    for (int h = 0; h < QH; ++h) exponentiate(s_cur[h], pk[h], h);   // VALU on S(j) ...
    compute_s(kst.template operator()<(R + 1) & 3>(), s_next);       // ... under MFMA S(j+1)
    compute_pv(vst.template operator()<R>(), pk);                    // MFMA O += V(j) P(j) ...
    float alpha[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) alpha[h] = new_reference(s_next[h], h);   // ... under the scan of S(j+1)
    rescale(alpha);
#pragma unroll
    for (int h = 0; h < QH; ++h)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s_cur[h][kt] = s_next[h][kt];
  };
  // Last unmasked iteration j = n_main - 1 (j % 4 == R).
  auto last_main = [&]<int R>(int j) {
    if (j + 1 < n_tiles) advance.template operator()<(R + 3) & 3>(j + 1);
#pragma unroll
    for (int h = 0; h < QH; ++h) exponentiate(s_cur[h], pk[h], h);
    compute_pv(vst.template operator()<R>(), pk);
  };
  // A tile that needs a mask (ragged tail; causal diagonal), t % 4 == R.
  // Rows with no allowed key in it get p = 0 exactly.
  auto masked = [&]<int R>(int t) {
    if (t > n_main || n_main == 0) advance.template operator()<(R + 2) & 3>(t);
    const int kv0 = t * C::BC;
    const bool active = (qw0 < p.Nq) && (!CAUSAL || kv0 <= qw0 + 32 * QH - 1);
    if (active) {
      f32x16 s[QH][KT];
      compute_s(kst.template operator()<R>(), s);
      float alpha[QH];
#pragma unroll
      for (int h = 0; h < QH; ++h) {
        const int myq = qw0 + 32 * h + l32;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            if ((key >= p.Nkv) || (CAUSAL && key > myq)) s[h][kt][r] = -INFINITY;
          }
        }
        alpha[h] = new_reference(s[h], h);
      }
      rescale(alpha);
#pragma unroll
      for (int h = 0; h < QH; ++h) exponentiate(s[h], pk[h], h);
      compute_pv(vst.template operator()<R>(), pk);
    }
  };

  if (n_main > 0) {
    advance.template operator()<2>(0);
    compute_s(kst.template operator()<0>(), s_cur);
    float alpha[QH];
#pragma unroll
    for (int h = 0; h < QH; ++h) alpha[h] = new_reference(s_cur[h], h);
    rescale(alpha);
    int j = 0;
    for (; j + 4 < n_main; j += 4) {
      steady.template operator()<0>(j);
      steady.template operator()<1>(j + 1);
      steady.template operator()<2>(j + 2);
      steady.template operator()<3>(j + 3);
    }
    for (; j + 1 < n_main; ++j) {
      switch (j & 3) {
        case 0: steady.template operator()<0>(j); break;
        case 1: steady.template operator()<1>(j); break;
        case 2: steady.template operator()<2>(j); break;
        default: steady.template operator()<3>(j); break;
      }
    }
    switch (j & 3) {
      case 0: last_main.template operator()<0>(j); break;
      case 1: last_main.template operator()<1>(j); break;
      case 2: last_main.template operator()<2>(j); break;
      default: last_main.template operator()<3>(j); break;
    }
  }
  for (int t = n_main; t < n_tiles; ++t) {
    switch (t & 3) {
      case 0: masked.template operator()<0>(t); break;
      case 1: masked.template operator()<1>(t); break;
      case 2: masked.template operator()<2>(t); break;
      default: masked.template operator()<3>(t); break;
    }
  }

  // Epilogue: combine the half-waves' sums, divide once, write O and lse.
  // Rows past N_q fall outside the buffer ranges and are dropped.
  const rsrc_t ro = make_rsrc(static_cast<uint16_t*>(p.o) + qhead * D, (uint32_t)p.Nq * C::ROWB);
  const rsrc_t rl = make_rsrc(p.lse + qhead, (uint32_t)p.Nq * 4u);
#pragma unroll
  for (int h = 0; h < QH; ++h) {
    const int myq = qw0 + 32 * h + l32;
    const float l_tot = pair_sum(l_run[h]);
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = M::pack(acc[h][db][4 * g] * inv, acc[h][db][4 * g + 1] * inv);
        w[1] = M::pack(acc[h][db][4 * g + 2] * inv, acc[h][db][4 * g + 3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, w), ro,
                                              (myq * D + db * 32 + g * 8 + half * 4) * 2, 0, 0);
      }
    }
    if (half == 0)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((m_run[h] + fast_log2(l_tot)) * kLn2), rl,
                                            myq * 4, 0, 0);
  }
}

template <int D>
constexpr int kNT16 = Cfg16<D>::NT;
template <int D>
constexpr int kWavesPerEU16 = Cfg16<D>::WAVES_PER_EU;

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(kNT16<D>)
    __attribute__((amdgpu_waves_per_eu(kWavesPerEU16<D>, kWavesPerEU16<D>)))
attn_fwd_mfma16(Params p) {
  attn_fwd_mfma16_body<T, D, CAUSAL>(p);
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
  if (d == 64) return {Cfg16<64>::BR, Cfg16<64>::BC, Cfg16<64>::NT, Cfg16<64>::LDS_BYTES};
  return {Cfg16<128>::BR, Cfg16<128>::BC, Cfg16<128>::NT, Cfg16<128>::LDS_BYTES};
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

template <typename T, int D, bool CAUSAL>
int run16(const Params& p, long long blocks, hipStream_t stream) {
  // All LDS of this kernel is static (one object per ring stage).
  return launch(attn_fwd_mfma16<T, D, CAUSAL>, 0, p, blocks, Cfg16<D>::NT, stream);
}

template <int D, bool CAUSAL>
int run32(const Params& p, long long blocks, hipStream_t stream) {
  using C = CfgF32<D>;
  static const int attr = set_lds_limit(attn_fwd_mfma_f32<D, CAUSAL>, C::LDS_BYTES);
  if (attr != FA_OK) return attr;
  return launch(attn_fwd_mfma_f32<D, CAUSAL>, C::LDS_BYTES, p, blocks, C::NT, stream);
}

template <typename T>
int dispatch16(const Params& p, int d, bool causal, long long blocks, hipStream_t s) {
  if (d == 64) return causal ? run16<T, 64, true>(p, blocks, s) : run16<T, 64, false>(p, blocks, s);
  return causal ? run16<T, 128, true>(p, blocks, s) : run16<T, 128, false>(p, blocks, s);
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
    case FA_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case FA_ERR_HIP: return g_hip_error[0] ? g_hip_error : "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
