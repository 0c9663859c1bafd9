// One MFMA GEMM core for every contraction of the path:
//     C[m, n] = sum_k A(m, k) * B(n, k)
// Each operand is either K-contiguous (element (p, k) at p*ld + k) or
// K-major (element (p, k) at k*ld + p). Three epilogues:
//   EPI_FWD   logits tile -> per-token (max, sum exp) over the tile's real
//             vocabulary rows + the target logit from the owning tile
//   EPI_GRAD  logits tile -> G = scale * (softmax - onehot), stored
//             token-major in the input element type
//   EPI_STORE plain float32 store / accumulate (dh and dW)
//   EPI_ARGMAX logits tile -> per-token (largest logit, lowest row index
//             holding it) over the tile's real vocabulary rows
//
// Workgroup: WAVES_M x WAVES_N waves over a BM x BN tile; each wave owns a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of 32 x 32 MFMA blocks (in bf16
// with two 128-byte stages, each is computed as four 16x16x32 blocks whose
// accumulators are rearranged into the 32x32 layout before the epilogue;
// their sums have come out bit-identical to the 32x32x16 ones, in less time
// per flop). K
// advances in slices of RB bytes per operand position (RB = 128: 64 bf16 or
// 32 float; 64 is supported too), staged in LDS by direct global->LDS loads
// (global_load_lds_dwordx4), NS stages deep; both layouts fill one stage with
// ROWS * RB bytes.
//
// K-contiguous stage: one RB-byte row per position, its 16-byte chunks
// permuted by ((row >> 1) & 7) (RB = 128) or ((row >> 2) & 3) (RB = 64) so
// that the 16 lanes one LDS cycle serves (16 consecutive rows, one chunk)
// cover all 64 banks. A fragment is one ds_read_b128 per lane.
//
// K-major stage: one row per K index holding the tile's positions. bf16
// fragments come from two ds_read_b64_tr_b16 per lane: within each group of
// 16 lanes the instruction hands lane i, element e, the element i % 4 of the
// 8 bytes that lane 4e + i/4 addressed; lane 4e + b of the group addresses
// row k + e at positions 4b..4b+3, so lane i receives four consecutive K
// values of position i. The 64-byte blocks of each 256-byte window of a row
// are permuted by (k & 3), and its 32-byte halves by bit 3 of k, so the rows
// one 32-lane pass reads (four, or two sets of four 8 apart in the 16x16x32
// form) fall on different banks. float fragments are four ds_read_b32; their rows k and
// k + 4 are separated by permuting 128-byte halves by ((k >> 2) & 1).
//
// Operand positions past the valid range read a clamped (valid) position and
// their results are discarded by the epilogues; K positions past K read zeros
// in whole 16-byte chunks (a row must therefore be readable up to its valid
// length rounded up to 16 bytes), so garbage never enters a valid sum.
//
// The M side can be cut into segments (the vocabulary shards, equal or not):
// tiles never cross a segment end, so every tile computes with one shard's rows.
#pragma once

#include <type_traits>

#include "vce_device.hpp"

// A second copy of the K loop for whole tiles, free of per-load tests
#ifndef VCE_KLOOP_SPLIT
#define VCE_KLOOP_SPLIT 1
#endif
// bf16 logit GEMMs (forward, G, argmax) on 16x16x32 MFMA blocks
#ifndef VCE_MFMA16
#define VCE_MFMA16 1
#endif
// The forward's epilogue reads the 16x16 accumulator blocks as they are (no
// rearrangement into the 32x32 layout)
#ifndef VCE_EPI16
#define VCE_EPI16 1
#endif
// Direct-to-LDS copies of each slice (of 8 per wave) that the logit GEMMs
// defer into the first MFMAs of the next slice: forward and argmax, G
#ifndef VCE_DMA_DEFER
#define VCE_DMA_DEFER 1
#endif
#ifndef VCE_DMA_DEFER_FWD
#define VCE_DMA_DEFER_FWD 6
#endif
#ifndef VCE_DMA_DEFER_GRAD
#define VCE_DMA_DEFER_GRAD 4
#endif

namespace vce {

enum EpiMode { EPI_FWD = 0, EPI_GRAD = 1, EPI_STORE = 2, EPI_ARGMAX = 3 };

struct GemmShape {
  const void* A;
  int64_t lda;          // elements between consecutive rows of A's storage
  const void* B;
  int64_t ldb;
  SegTable seg;         // M segments (vocabulary shards) and their tiles
  int64_t m_total;      // tile ends are clipped to this
  int64_t m_load_end;   // A positions at or past this are never read
  int64_t n_total;      // B positions at or past this are never read
  int32_t tiles_n;
  int32_t k_splits;     // split of K into independent partial products
  int64_t k_total;      // K extent; K positions at or past it read as zero
  int64_t k_per_split;  // multiple of the K slice
  int32_t group_m;      // tiles along M visited together by one XCD
};

struct FwdArgs {
  const int32_t* targets;
  int64_t T;
  int64_t V_real;
  float2* stats;        // [tiles_m][T]: (max, sum exp(z - max)) of every tile
  float* zt;            // [T]: target logit, written by the owning tile only
};

struct GradArgs {
  const int32_t* targets;
  const float* lse;
  int64_t T;
  int64_t V_real;
  const float* grad_loss;
  const int32_t* n_valid;
  int64_t v_off;        // vocabulary row of the GEMM's row 0
  int32_t reduction;    // 0 mean over valid tokens, 1 sum
  int32_t vec_store;    // 1 if tile rows start at multiples of 8 and ldG is one (16-byte stores)
  void* G;              // [T][ldG]
  int64_t ldG;
};

struct StoreArgs {
  float* C;
  int64_t ldc;
  float* P;             // K splits 1, 2, ...: partial planes [k_splits - 1][M][ldc]
  int64_t split_stride; // elements between partial planes
  int32_t accumulate;   // split 0: 1: C += result, 0: C = result
  int32_t planes_held;  // planes below this index already hold a sum: added to, the others overwritten
  int64_t m_zero_from;  // rows at or past this receive 0 (or are left alone when accumulating)
};

struct ArgArgs {
  int64_t T;
  float* val;           // [tiles_m][T]: largest logit of the tile's real rows (-inf if none)
  int32_t* idx;         // [tiles_m][T]: its vocabulary row, the lowest on ties (-1 if none)
};

struct EpiArgs {
  FwdArgs fwd;
  GradArgs grad;
  StoreArgs store;
  ArgArgs arg;
};

// 16 zero bytes: the source of the chunks that lie past K
static __device__ __attribute__((aligned(64))) const uint32_t g_zero_chunk[16] = {0};

template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 bits
  static constexpr int kSlice = 64;  // K elements per 128-byte slice
  static constexpr int kChunk = 8;   // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int kSlice = 32;
  static constexpr int kChunk = 4;
};

// s_waitcnt vmcnt(N) with the other counters left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses are done
// (lgkmcnt(0)), outstanding global loads are left in flight. __syncthreads()
// would also wait for every global load, including the next tile's prefetch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
  __builtin_amdgcn_s_barrier();
}

template <typename E>
__device__ __forceinline__ void mma_chunk(f32x16& acc, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mma_chunk<uint16_t>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// bf16 on 16x16x32 blocks (16x16 layout: lane l holds column l % 16, rows
// 4 (l / 16) .. +3 of the block)
__device__ __forceinline__ void mma16(f32x4& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                              __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Four 16x16 blocks b[ra][cb] (rows 16 ra + .., columns 16 cb + ..) -> one
// 32 x 32 block in the 32x32 layout (lane l: column l % 32, register 4q + r:
// row 8q + 4 (l / 32) + r). That element sits in block (q / 2, l / 16 % 2) at
// row 8 (q % 2) + 4 (l / 32) + r, i.e. in register r of lane
// l % 16 + 16 (2 (q % 2) + l / 32). For fixed ra and r, with P, Q the
// registers of blocks (ra, 0) and (ra, 1) and rows counted in 16-lane groups,
// the outputs q = 2 ra and 2 ra + 1 are [P0 Q0 P1 Q1] and [P2 Q2 P3 Q3]: a
// 16-lane swap (odd groups of the first operand with even groups of the
// second: [P0 Q0 P2 Q2], [P1 Q1 P3 Q3]) followed by a 32-lane swap (upper half
// of the first with lower half of the second).
__device__ __forceinline__ void rows32_layout(f32x16& out, const f32x4& b00, const f32x4& b01,
                                              const f32x4& b10, const f32x4& b11) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const auto p0 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b00[r]), __float_as_uint(b01[r]),
                                                     false, false);
    const auto q0 = __builtin_amdgcn_permlane32_swap(p0[0], p0[1], false, false);
    out[r] = __uint_as_float(q0[0]);
    out[4 + r] = __uint_as_float(q0[1]);
    const auto p1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(b10[r]), __float_as_uint(b11[r]),
                                                     false, false);
    const auto q1 = __builtin_amdgcn_permlane32_swap(p1[0], p1[1], false, false);
    out[8 + r] = __uint_as_float(q1[0]);
    out[12 + r] = __uint_as_float(q1[1]);
  }
}

// float32: the lane's 4 floats are 4 K positions; one 32x32x2 MFMA per
// component (lanes 0-31 give one K position, lanes 32-63 another). A and B
// use the same assignment, so the four products cover the 8 K values of a
// sub-step once each.
template <>
__device__ __forceinline__ void mma_chunk<float>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// 32-bit LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(p)));
}

// Global -> LDS copy of one 16-byte chunk per lane, landing at LDS address
// lds + 16 * lane (global_load_lds_dwordx4). Written as inline assembly on
// purpose: the compiler cannot tell which LDS bytes such a load writes, so
// for its own intrinsic it waits for every outstanding load before any later
// LDS read, which would wait for the next slice's prefetch before computing
// on the current one. The kernel orders these copies itself (s_waitcnt
// vmcnt + s_barrier); the compiler only has to keep LDS accesses on their side
// of the statement, which the memory clobber does. M0 is written here and the
// compiler keeps nothing in M0 across these kernels' code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// address = 64-bit scalar base + 32-bit per-lane offset
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// address = per-lane 64-bit pointer
__device__ __forceinline__ void dma16(const void* p, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(p), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// ---------------------------------------------------------------- stagers
// A stager brings one operand's K slice of one tile into an LDS stage and
// reads MFMA fragments out of it. ROWS = positions of the tile (BM or BN),
// NW = waves of the workgroup. Interface:
//   init<NB>(p0, p_end, ld, wave, lane, wbase)
//        tile positions [p0, p_end) are valid; the wave's fragments cover NB
//        blocks of 32 positions from tile position wbase
//   fast(kleft)                     all rows valid and a whole slice left
//   issue_q(q, lds, base, kleft, wave, fast)
//                                   load q (of Q) of one slice; base =
//                                   element (p0, k); kleft = K left
//   issue(lds, base, kleft, wave)   all Q loads of one slice
//   frag(stage, block, s, lane)     fragment of one block at sub-step s
//                                   (16 bf16 / 8 float of K)
//   kReads                          LDS read instructions per fragment

// K-contiguous operand; RB = bytes of one position's K slice (128 or 64)
template <typename E, int ROWS, int NW, int RB>
struct StageKC {
  static constexpr int ES = sizeof(E);
  static constexpr int EPC = Elem<E>::kChunk;
  static constexpr int BK = RB / ES;      // K elements per slice
  static_assert(RB == 128 || RB == 64, "slice bytes");
  static constexpr int CPR = RB / 16;     // chunks per row
  static constexpr int RPI = 64 / CPR;    // rows per wave-wide load
  static constexpr int Q = ROWS / (RPI * NW);
  static constexpr int kReads = 1;
  static_assert(ROWS % (RPI * NW) == 0, "load split");
  static_assert(RB == 64 || NW % 2 == 0, "chunk choice must not depend on the load index");
  uint32_t off0;     // this lane's byte offset for load 0 (chunk included)
  int32_t lrow;      // this lane's tile row for load 0
  int32_t kch;       // element offset of this lane's chunk inside the K slice
  int32_t nrows;     // valid rows of the tile
  int64_t rstride;   // bytes between consecutive rows
  uint32_t frag0;    // this lane's LDS row offset for block 0

  // 16 lanes of one LDS cycle read 16 consecutive rows at one logical chunk;
  // the permutation spreads them over all 64 banks
  __device__ __forceinline__ static int swz(int row) {
    return RB == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3);
  }

  template <int NB>
  __device__ __forceinline__ void init(int64_t p0, int64_t p_end, int64_t ld, int wave, int lane,
                                       int wbase) {
    lrow = wave * RPI + lane / CPR;
    const int lch = (lane % CPR) ^ swz(lrow);
    kch = lch * EPC;
    rstride = ld * ES;
    nrows = static_cast<int32_t>(min(p_end - p0, static_cast<int64_t>(ROWS)));
    off0 = static_cast<uint32_t>(lrow * rstride + kch * ES);
    frag0 = static_cast<uint32_t>((wbase + (lane & 31)) * RB);
  }

  __device__ __forceinline__ bool fast(int64_t kleft) const { return kleft >= BK && nrows == ROWS; }

  __device__ __forceinline__ void issue_q(int q, uint32_t lds, const char* base, int64_t kleft,
                                          int wave, bool is_fast) const {
    const uint32_t dst = lds + (q * NW + wave) * RPI * RB;
    if (is_fast) {
      dma16(base + q * (static_cast<int64_t>(NW) * RPI * rstride), off0, dst);
    } else {
      // recomputed at every use (the empty asm hides that lr is invariant):
      // kept live across the K loop, these addresses would cost registers
      int lr = lrow;
      asm volatile("" : "+v"(lr));
      int r = lr + q * NW * RPI;
      if (r >= nrows) r = nrows - 1;  // the result of this row is discarded
      const void* p = base + static_cast<uint32_t>(r * static_cast<int32_t>(rstride) + kch * ES);
      if (kch >= kleft) p = g_zero_chunk;
      dma16(p, dst);
    }
  }

  __device__ __forceinline__ void issue(uint32_t lds, const char* base, int64_t kleft,
                                        int wave) const {
    const bool f = fast(kleft);
#pragma unroll
    for (int q = 0; q < Q; ++q) issue_q(q, lds, base, kleft, wave, f);
  }

  // fragment: row (wbase + block*32 + lane%32), logical chunk 2s + lane/32
  // (the rows of a block start at a multiple of 32, so swz depends on lane%32)
  __device__ __forceinline__ u32x4 frag(const char* st, int block, int s, int lane) const {
    const int ch = ((2 * s + (lane >> 5)) ^ swz(lane & 31)) * 16;
    return *reinterpret_cast<const u32x4*>(st + frag0 + block * 32 * RB + ch);
  }

  // 16x16x32 fragment (RB = 128): row (wbase + 16 grp + lane % 16), logical
  // chunk 4 sub + lane / 16 (a group starts at a multiple of 16 rows)
  uint32_t f16;  // this lane's row offset for group 0
  int32_t s16;   // its row's chunk permutation
  __device__ __forceinline__ void init16(int wbase, int lane) {
    f16 = static_cast<uint32_t>((wbase + (lane & 15)) * RB);
    s16 = swz(lane & 15);
  }
  __device__ __forceinline__ u32x4 frag16(const char* st, int grp, int sub, int lane) const {
    const int ch = ((4 * sub + (lane >> 4)) ^ s16) * 16;
    return *reinterpret_cast<const u32x4*>(st + f16 + grp * 16 * RB + ch);
  }
};

// K-major operand; a slice holds RB / sizeof(E) K rows
template <typename E, int ROWS, int NW, int RB>
struct StageKM {
  static constexpr int ES = sizeof(E);
  static constexpr int EPC = Elem<E>::kChunk;
  static constexpr int BK = RB / ES;           // K rows per slice
  static constexpr int RBT = ROWS * ES;        // bytes per K row of the tile
  static constexpr int RPL = 1024 / RBT;       // K rows per wave-wide load
  static constexpr int CPR = RBT / 16;         // chunks per K row
  static constexpr int Q = BK / (RPL * NW);
  static constexpr int kReads = ES == 2 ? 2 : 4;
  static_assert(1024 % RBT == 0 && RBT >= 256, "row size");
  static_assert(BK % (RPL * NW) == 0 && Q >= 1, "load split");
  // the chunk permutation repeats every 16 (bf16) / 8 (float) rows: when the
  // rows of consecutive loads step by a multiple of that, a lane's chunk is
  // the same for every load
  static constexpr bool kQIndep = (RPL * NW) % (ES == 2 ? 16 : 8) == 0;
  uint32_t off0;     // this lane's byte offset for load 0 (chunk included)
  int32_t lk;        // this lane's K row (within the slice) for load 0
  int32_t pch;       // this lane's chunk slot in its LDS row
  int32_t lch;       // the logical chunk (of positions) it brings for load 0
  int32_t last_ch;   // last chunk holding a valid position
  bool all_cols;
  int64_t rstride;   // bytes between consecutive K rows in global memory
  uint32_t fb[4];    // this lane's LDS byte offset of each block's fragment (sub-step 0)

  // permutation of the chunks of K row k
  __device__ __forceinline__ static int swz(int k) {
    return ES == 2 ? (((k & 3) << 2) ^ (((k >> 3) & 1) << 1)) : (((k >> 2) & 1) << 3);
  }

  template <int NB>
  __device__ __forceinline__ void init(int64_t p0, int64_t p_end, int64_t ld, int wave, int lane,
                                       int wbase) {
    static_assert(NB <= 4, "fragment offsets");
    lk = wave * RPL + lane / CPR;
    pch = lane % CPR;
    lch = pch ^ swz(lk);
    rstride = ld * ES;
    const int64_t npos = min(p_end - p0, static_cast<int64_t>(ROWS));
    all_cols = npos == ROWS;
    last_ch = static_cast<int32_t>((npos - 1) / EPC);
    off0 = static_cast<uint32_t>(lk * rstride + lch * 16);
    if constexpr (ES == 2) {
      const int i = lane & 15, g = (lane >> 4) & 1, hk = lane >> 5;
      const int krow = 8 * hk + (i >> 2);  // row within the sub-step for read 0
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int pos = wbase + b * 32 + 16 * g + 4 * (i & 3);
        const int ch = (pos / EPC) ^ swz(krow);
        fb[b] = static_cast<uint32_t>(krow * RBT + ch * 16 + (pos % EPC) * ES);
      }
    } else {
      const int l32 = lane & 31, half = lane >> 5;
      const int krow = 4 * half;           // row within the sub-step for component 0
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int pos = wbase + b * 32 + l32;
        const int ch = (pos / EPC) ^ swz(krow);
        fb[b] = static_cast<uint32_t>(krow * RBT + ch * 16 + (pos % EPC) * ES);
      }
    }
  }

  __device__ __forceinline__ bool fast(int64_t kleft) const {
    return kQIndep && kleft >= BK && all_cols;
  }

  __device__ __forceinline__ void issue_q(int q, uint32_t lds, const char* base, int64_t kleft,
                                          int wave, bool is_fast) const {
    const uint32_t dst = lds + (q * NW + wave) * 1024;
    if (is_fast) {
      dma16(base + q * (static_cast<int64_t>(NW) * RPL * rstride), off0, dst);
    } else {
      int l0 = lk;  // recomputed at every use, as in StageKC
      asm volatile("" : "+v"(l0));
      const int k = l0 + q * NW * RPL;
      const int ch = kQIndep ? lch : (pch ^ swz(k));
      const int c = min(ch, last_ch);  // positions past the valid range: discarded
      const void* p = base + static_cast<uint32_t>(k * static_cast<int32_t>(rstride) + c * 16);
      if (k >= kleft) p = g_zero_chunk;
      dma16(p, dst);
    }
  }

  __device__ __forceinline__ void issue(uint32_t lds, const char* base, int64_t kleft,
                                        int wave) const {
    const bool f = fast(kleft);
#pragma unroll
    for (int q = 0; q < Q; ++q) issue_q(q, lds, base, kleft, wave, f);
  }

  __device__ __forceinline__ u32x4 frag(const char* st, int block, int s, int lane) const {
    (void)lane;
    const char* p = st + fb[block];
    if constexpr (ES == 2) {
      // read r covers K rows 16s + 8hk + 4r + (0..3); rows 4 apart share the
      // chunk permutation, so read 1 is read 0 four rows further
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * s * RBT));
      const s16x4 r1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (16 * s + 4) * RBT));
      const u32x2 a = __builtin_bit_cast(u32x2, r0), b = __builtin_bit_cast(u32x2, r1);
      return u32x4{a.x, a.y, b.x, b.y};
    } else {
      // component c: K row 8s + 4*half + c (the permutation depends on half only)
      u32x4 v;
      v.x = *(const lds_u32*)(p + (8 * s + 0) * RBT);
      v.y = *(const lds_u32*)(p + (8 * s + 1) * RBT);
      v.z = *(const lds_u32*)(p + (8 * s + 2) * RBT);
      v.w = *(const lds_u32*)(p + (8 * s + 3) * RBT);
      return v;
    }
  }

  // 16x16x32 fragment (bf16): position wbase + 16 grp + lane % 16, K rows
  // 32 sub + 8 (lane / 16) + 0..7 from two transposing reads of four rows.
  // Lane 4e + b of each 16-lane group addresses row +e, positions 4b..4b+3;
  // a 32-lane pass covers rows 8q + 0..3 of two groups q, which the
  // permutation's bit from row bit 3 puts on other banks.
  uint32_t f16;  // this lane's row offset (read 0, sub-step 0) plus its element offset
  int32_t c16;   // its unpermuted chunk for group 0
  int32_t s16;   // its rows' chunk permutation
  __device__ __forceinline__ void init16(int wbase, int lane) {
    const int i = lane & 15, q = lane >> 4;
    const int krow = 8 * q + (i >> 2);
    const int pos = wbase + 4 * (i & 3);
    f16 = static_cast<uint32_t>(krow * RBT + (pos % EPC) * ES);
    c16 = pos / EPC;
    s16 = swz(krow);
  }
  __device__ __forceinline__ u32x4 frag16(const char* st, int grp, int sub, int lane) const {
    (void)lane;
    if constexpr (ES == 2) {
      const char* p = st + f16 + 32 * sub * RBT + ((c16 + 2 * grp) ^ s16) * 16;
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * RBT));
      const u32x2 a = __builtin_bit_cast(u32x2, r0), b = __builtin_bit_cast(u32x2, r1);
      return u32x4{a.x, a.y, b.x, b.y};
    } else {
      return u32x4{0u, 0u, 0u, 0u};  // the 16x16x32 form is bf16 only
    }
  }
};

template <typename E, int ROWS, int NW, int RB, bool KMAJ>
using Stager =
    typename std::conditional<KMAJ, StageKM<E, ROWS, NW, RB>, StageKC<E, ROWS, NW, RB>>::type;

// Compile-time loop: f(integral_constant<int, I>) for I in [I0, N)
template <int I0, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I0 < N) {
    f(std::integral_constant<int, I0>{});
    static_for<I0 + 1, N>(f);
  }
}

// Geometry of one output tile.
struct TileGeom {
  int64_t tm;      // tile index along M (segment-major)
  int64_t ks;      // K split
  int64_t m0, m_end, m_load, n0, n_end, k_beg, k_end;
  __device__ __forceinline__ bool active() const {
    return m_load > m0 && n_end > n0 && k_end > k_beg;
  }
};

// Logical tile L -> tile: K split outermost, then groups of group_m tiles
// along M, each group walking all tiles along N. Tile counts fit in 32 bits
// (checked on the host), so the divisions are 32-bit.
template <int BM, int BN>
__device__ __forceinline__ TileGeom decode_tile(const GemmShape& g, uint32_t L) {
  const uint32_t tiles_m = static_cast<uint32_t>(g.seg.tile[g.seg.n]);
  const uint32_t tiles_n = static_cast<uint32_t>(g.tiles_n);
  const uint32_t group_m = static_cast<uint32_t>(g.group_m);
  const uint32_t per_split = tiles_m * tiles_n;
  TileGeom t;
  const uint32_t ks = L / per_split;
  const uint32_t rem = L - ks * per_split;
  const uint32_t in_group = group_m * tiles_n;
  const uint32_t grp = rem / in_group;
  const uint32_t first_m = grp * group_m;
  const uint32_t gsz = min(group_m, tiles_m - first_m);
  const uint32_t r_in = rem - grp * in_group;
  const uint32_t tn = r_in / gsz;
  const uint32_t tm = first_m + (r_in - tn * gsz);
  const int seg = shard_of_tile(g.seg, tm);
  const uint32_t tj = tm - static_cast<uint32_t>(g.seg.tile[seg]);
  t.ks = ks;
  t.tm = tm;
  t.m0 = g.seg.row[seg] + static_cast<int64_t>(tj) * BM;
  t.m_end = min(min(t.m0 + BM, g.seg.row[seg + 1]), g.m_total);
  t.m_load = min(t.m_end, g.m_load_end);
  t.n0 = static_cast<int64_t>(tn) * BN;
  t.n_end = min(t.n0 + static_cast<int64_t>(BN), g.n_total);
  t.k_beg = static_cast<int64_t>(ks) * g.k_per_split;
  t.k_end = min(t.k_beg + g.k_per_split, g.k_total);
  return t;
}

// Persistent GEMM: the grid holds a multiple of 8 workgroups (one per CU).
// Workgroups are handed to the 8 XCDs round-robin, so the workgroups of one
// XCD (blockIdx % 8 equal) take one contiguous range of logical tiles and walk
// it together, sharing operand tiles in that XCD's L2. While a tile's
// epilogue runs, the first K slices of the workgroup's next tile are already
// on their way into LDS.
template <typename E, int MODE, bool AKM, bool BKM, int BM, int BN, int WAVES_M, int WAVES_N,
          int RB, int NS, int OCC, bool SPREAD>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES_M * WAVES_N,
                                                      64 * WAVES_M * WAVES_N),
                          amdgpu_waves_per_eu(OCC, OCC)))
void k_gemm_tn(GemmShape g, EpiArgs e) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int ES = sizeof(E);
  constexpr int BK = RB / ES;              // K elements per slice
  constexpr int SS = RB / 32;              // sub-steps per slice (16 bf16 / 8 float of K each)
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(NS >= 2 && SS >= 2 && SS % 2 == 0, "stages");
  static_assert(!SPREAD || NS >= 3, "spread issue needs a free stage ahead");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  __shared__ float2 red[MODE == EPI_FWD && WAVES_M > 1    ? (WAVES_M - 1) * BN
                      : MODE == EPI_ARGMAX && WAVES_M > 1 ? WAVES_M * BN
                                                          : 1];

  using SA = Stager<E, BM, NW, RB, AKM>;
  using SB = Stager<E, BN, NW, RB, BKM>;
  constexpr int LOADS = SA::Q + SB::Q;  // VMEM instructions per slice per wave
  if constexpr (MI * NI * 16 > 128) {
    // Accumulators above half the register file: naming an accumulation
    // register keeps the compiler from assuming the kernel uses none, so it
    // selects the MFMA forms that accumulate in AGPRs instead of copying
    // between the two register files.
    asm volatile("" ::: "a0");
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- this workgroup's tiles: L = start + wi, start + wi + per_xcd, ... < end
  const uint32_t total = static_cast<uint32_t>(g.seg.tile[g.seg.n]) *
                         static_cast<uint32_t>(g.tiles_n) * static_cast<uint32_t>(g.k_splits);
  const uint32_t xcd = blockIdx.x & 7;
  const uint32_t wi = blockIdx.x >> 3;
  const uint32_t per_xcd = gridDim.x >> 3;
  const uint32_t q8 = total >> 3, r8 = total & 7;
  const uint32_t start = xcd * q8 + min(xcd, r8);
  const uint32_t end = start + q8 + (xcd < r8 ? 1u : 0u);
  uint32_t L = start + wi;
  if (L >= end) return;

  // per-tile load state
  SA sa;
  SB sb;
  const char* Ab = nullptr;
  const char* Bb = nullptr;
  int64_t klen = 0;
  int nk = 0;
  auto setup = [&](const TileGeom& t) {
    sa.template init<MI>(t.m0, t.m_load, g.lda, wave, lane, wm * WM);
    sb.template init<NI>(t.n0, t.n_end, g.ldb, wave, lane, wn * WN);
    if constexpr (AKM)
      Ab = static_cast<const char*>(g.A) + (t.k_beg * g.lda + t.m0) * ES;
    else
      Ab = static_cast<const char*>(g.A) + (t.m0 * g.lda + t.k_beg) * ES;
    if constexpr (BKM)
      Bb = static_cast<const char*>(g.B) + (t.k_beg * g.ldb + t.n0) * ES;
    else
      Bb = static_cast<const char*>(g.B) + (t.n0 * g.ldb + t.k_beg) * ES;
    klen = t.k_end - t.k_beg;
    nk = t.active() ? static_cast<int>((klen + BK - 1) / BK) : 0;
  };

  const uint32_t smem_lds = lds_addr(smem);
  auto issue = [&](int kt) {
    const uint32_t st = smem_lds + (kt % NS) * STAGE;
    const int64_t kofs = static_cast<int64_t>(kt) * BK;
    const int64_t kleft = klen - kofs;
    sa.issue(st, Ab + kofs * (AKM ? g.lda : 1) * ES, kleft, wave);
    sb.issue(st + A_BYTES, Bb + kofs * (BKM ? g.ldb : 1) * ES, kleft, wave);
  };
  auto prologue = [&]() {
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
      if (p < nk) issue(p);
    asm volatile("" ::"r"(smem) : "memory");
  };

  // loss scaling of G, read once before any loads are in flight
  float scale = 0.0f;
  if constexpr (MODE == EPI_GRAD) {
    const float gl = e.grad.grad_loss[0];
    scale = (e.grad.reduction == 0) ? gl / static_cast<float>(max(e.grad.n_valid[0], 1)) : gl;
  }

  TileGeom cur = decode_tile<BM, BN>(g, L);
  setup(cur);
  prologue();

  // Per-token epilogue inputs of the current tile. Loaded during its first K
  // slice, so the explicit vmcnt waits of the K loop cover them and the
  // epilogue needs no wait of its own (which would also wait for the next
  // tile's prefetch).
  // bf16 on 16x16x32 blocks (two 128-byte stages); the forward's epilogue
  // then works on the 16 x 16 blocks directly (E16), whose lane l holds
  // column l % 16 of its block: 2 NI token columns per lane (measured 0.9 %
  // faster than rearranging them; the argmax kept the rearrangement, 0.6 %
  // faster with it)
  constexpr bool M16 = VCE_MFMA16 && sizeof(E) == 2 && RB == 128 && NS == 2 && !SPREAD;
  constexpr bool E16 = M16 && VCE_EPI16 && MODE == EPI_FWD;
  constexpr int NCOL = E16 ? 2 * NI : NI;
  int32_t yv[NCOL];
  float lv[NCOL];
  auto load_epi = [&]() {
#pragma unroll
    for (int j = 0; j < NCOL; ++j) {
      const int64_t tt =
          cur.n0 + wn * WN + (E16 ? j * 16 + (lane & 15) : j * 32 + l32);
      yv[j] = -1;
      lv[j] = 0.0f;
      if constexpr (MODE == EPI_FWD) {
        if (tt < e.fwd.T) yv[j] = e.fwd.targets[tt];
      } else if constexpr (MODE == EPI_GRAD) {
        if (tt < e.grad.T) {
          yv[j] = e.grad.targets[tt];
          lv[j] = e.grad.lse[tt];
        }
      }
    }
  };

  // Fragment reads of one sub-step and the MFMAs of one sub-step.
  auto read_frags = [&](const char* st, int sub, u32x4 (&fa)[MI], u32x4 (&fb)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = sa.frag(st, i, sub, lane);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = sb.frag(st + A_BYTES, j, sub, lane);
  };
  constexpr int NF = MI * SA::kReads + NI * SB::kReads;    // LDS reads per sub-step
  constexpr int NMF = MI * NI * (sizeof(E) == 2 ? 1 : 4);  // MFMAs per sub-step
  // scheduling hint: the next sub-step's NF reads spread evenly over this
  // sub-step's NMF MFMAs
  auto interleave = [&]() {
    static_for<0, NMF>([&](auto kk) {
      constexpr int k = decltype(kk)::value;
      constexpr int nd = (NF * (k + 1)) / NMF - (NF * k) / NMF;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nd, 0);
    });
  };

  f32x16 acc[MI][NI];
  u32x4 fa[2][MI], fb[2][NI];

  // 16x16x32 form (bf16, two 128-byte stages): A in groups of 16 rows, B in
  // groups of 16 columns, K = 32 per sub-step (two per slice); a lane's
  // fragment is position lane % 16 of its group, K values 8 (lane / 16) ..+7
  // of the sub-step (the stagers' frag16).
  constexpr int MA = 2 * MI, NB = 2 * NI, SS16 = RB / 64;
  if constexpr (M16) {
    sa.init16(wm * WM, lane);
    sb.init16(wn * WN, lane);
  }
  u32x4 Ar[4], B16[M16 ? NB : 1];
  f32x4 acc16[M16 ? MA : 1][M16 ? NB : 1];
  static_assert(!M16 || (SS16 == 2 && MA % 4 == 0 && LOADS <= 2 * NB), "16x16x32 slice geometry");

  while (true) {
    if constexpr (M16) {
#pragma unroll
      for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc16[a][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    }
    auto mfmas = [&](const u32x4 (&a)[MI], const u32x4 (&b)[NI]) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) mma_chunk<E>(acc[i][j], a[i], b[j]);
    };

    // Software pipeline over K slices. The prologue has queued slices
    // 0 .. NS-2. Slice kt+1's barrier sits before slice kt's last sub-step,
    // whose fragments are already in registers: its MFMAs cover the barrier
    // and the reads of slice kt+1's first fragments. Right after that barrier
    // every wave is done reading slice kt, so slice kt+NS is queued into its
    // stage; NS-1 slices are then in flight while one is consumed.
    //   WAIT_ALL: wait for every load (near the end, fewer slices are younger)
    //   ISSUE:    queue slice kt + NS
    //   LAST:     the tile's last slice (no barrier, nothing more to read)
    //   AF:       every slice of the tile is whole (all positions valid, K a
    //             multiple of the slice): the loads take the fast form with
    //             no run-time test
    auto kstep = [&](int kt, auto wait_all, auto issue_next, auto last, auto all_fast) {
      constexpr bool WAIT_ALL = decltype(wait_all)::value;
      constexpr bool ISSUE = decltype(issue_next)::value;
      constexpr bool LAST = decltype(last)::value;
      constexpr bool AF = decltype(all_fast)::value;
      const char* st = smem + (kt % NS) * STAGE;
      if constexpr (SPREAD && ISSUE) {
        // slice kt+NS-1 goes into the stage slice kt-1 used (free since the
        // previous barrier); its loads are spread over the MFMAs of the
        // sub-steps before this slice's barrier
        const int kn = kt + NS - 1;
        const int64_t kofs = static_cast<int64_t>(kn) * BK;
        const uint32_t stl = smem_lds + (kn % NS) * STAGE;
        const int64_t kleft = klen - kofs;
        const char* pa = Ab + kofs * (AKM ? g.lda : 1) * ES;
        const char* pb = Bb + kofs * (BKM ? g.ldb : 1) * ES;
        const bool fast_a = AF || sa.fast(kleft), fast_b = AF || sb.fast(kleft);
        constexpr int NT = MI * NI;
        constexpr int SLOTS = (SS - 1) * NT;  // MFMAs before the barrier
        static_for<0, SS - 1>([&](auto ss) {
          constexpr int sub = decltype(ss)::value;
          read_frags(st, sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
          static_for<0, NT>([&](auto kk) {
            constexpr int k = decltype(kk)::value;
            constexpr int slot = sub * NT + k;
            // loads l with l * SLOTS / LOADS == slot go right before this MFMA
            bool loaded = false;
            static_for<0, LOADS>([&](auto ll) {
              constexpr int l = decltype(ll)::value;
              if constexpr ((l * SLOTS) / LOADS == slot) {
                if constexpr (l < SA::Q)
                  sa.issue_q(l, stl, pa, kleft, wave, fast_a);
                else
                  sb.issue_q(l - SA::Q, stl + A_BYTES, pb, kleft, wave, fast_b);
                loaded = true;
              }
            });
            mma_chunk<E>(acc[k / NI][k % NI], fa[sub & 1][k / NI], fb[sub & 1][k % NI]);
            // as below: keep the loads where they were placed
            if (AF && loaded) __builtin_amdgcn_sched_barrier(0);
          });
        });
      } else {
#pragma unroll
        for (int sub = 0; sub + 1 < SS; ++sub) {
          read_frags(st, sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
          mfmas(fa[sub & 1], fb[sub & 1]);
          interleave();
        }
      }
      constexpr int LB = (SS - 1) & 1;
      if constexpr (!LAST) {
        // this wave's reads of slice kt are complete, its part of slice kt+1 is in
        __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
        if constexpr (WAIT_ALL)
          wait_vmcnt<0>();
        else
          wait_vmcnt<(NS - 2) * LOADS>();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::"r"(smem) : "memory");
        // The last sub-step's MFMAs, each followed by one load of slice kt+NS
        // and, in turn, the next slice's first fragment reads.
        const char* stn = smem + ((kt + 1) % NS) * STAGE;
        const char *pa = nullptr, *pb = nullptr;
        uint32_t stl = 0;
        int64_t kleft = 0;
        bool fast_a = true, fast_b = true;
        if constexpr (ISSUE && !SPREAD) {
          const int kn = kt + NS;
          const int64_t kofs = static_cast<int64_t>(kn) * BK;
          stl = smem_lds + (kn % NS) * STAGE;
          kleft = klen - kofs;
          pa = Ab + kofs * (AKM ? g.lda : 1) * ES;
          pb = Bb + kofs * (BKM ? g.ldb : 1) * ES;
          fast_a = AF || sa.fast(kleft);
          fast_b = AF || sb.fast(kleft);
        }
        constexpr int NT = MI * NI;
        static_for<0, (NT > LOADS ? NT : LOADS)>([&](auto kk) {
          constexpr int k = decltype(kk)::value;
          if constexpr (ISSUE && !SPREAD && k < LOADS) {
            if constexpr (k < SA::Q)
              sa.issue_q(k, stl, pa, kleft, wave, fast_a);
            else
              sb.issue_q(k - SA::Q, stl + A_BYTES, pb, kleft, wave, fast_b);
          }
          if constexpr (k < NT) mma_chunk<E>(acc[k / NI][k % NI], fa[LB][k / NI], fb[LB][k % NI]);
          if constexpr (k < MI)
            fa[0][k] = sa.frag(stn, k, 0, lane);
          else if constexpr (k < MI + NI)
            fb[0][k - MI] = sb.frag(stn + A_BYTES, k - MI, 0, lane);
          // keep one load per MFMA: without run-time tests around the loads
          // the scheduler would otherwise hoist them all ahead of the MFMAs
          if constexpr (AF && ISSUE) __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (NT < MI + NI) {
#pragma unroll
          for (int k = NT; k < MI + NI; ++k) {
            if (k < MI)
              fa[0][k] = sa.frag(stn, k, 0, lane);
            else
              fb[0][k - MI] = sb.frag(stn + A_BYTES, k - MI, 0, lane);
          }
        }
      } else {
        mfmas(fa[LB], fb[LB]);
      }
    };

    // The same pipeline on 16x16x32 blocks. A sub-step runs A group by A
    // group; the A fragments live in a ring of four, group a+2's read before
    // group a's MFMAs (from this sub-step's source, or from the next
    // sub-step's once a+2 passes the last group), and each B fragment is read
    // again for the next sub-step right after its last MFMA (in the last
    // group). In a slice's second sub-step the reads of the next slice start
    // at group MA-2, so slice kt+1's wait and barrier sit there (mid), and the
    // copies of slice kt+NS go out among the last two groups' MFMAs (dma) or,
    // those the logit GEMMs defer, among the next slice's first MFMAs (dma0).
    auto sub16 = [&](const char* stc, int sc, const char* stx, int sx, auto next, auto mid,
                     auto dma) {
      constexpr bool NX = decltype(next)::value;
      static_for<0, MA>([&](auto aa) {
        constexpr int a = decltype(aa)::value;
        if constexpr (a == MA - 2) mid();
        if constexpr (a + 2 < MA)
          Ar[(a + 2) % 4] = sa.frag16(stc, a + 2, sc, lane);
        else if constexpr (NX)
          Ar[(a + 2) % 4] = sa.frag16(stx, a + 2 - MA, sx, lane);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NB>([&](auto bb) {
          constexpr int b = decltype(bb)::value;
          dma(std::integral_constant<int, a * NB + b>{});
          mma16(acc16[a][b], Ar[a % 4], B16[b]);
          if constexpr (NX && a == MA - 1) B16[b] = sb.frag16(stx + A_BYTES, b, sx, lane);
          __builtin_amdgcn_sched_barrier(0);
        });
      });
    };
    auto read16 = [&](const char* st) {
      Ar[0] = sa.frag16(st, 0, 0, lane);
      Ar[1] = sa.frag16(st, 1, 0, lane);
#pragma unroll
      for (int b = 0; b < NB; ++b) B16[b] = sb.frag16(st + A_BYTES, b, 0, lane);
    };
    // The copies of one slice: in the logit GEMMs, LH of them go out among
    // the MFMAs after the barrier that frees their stage (every other one)
    // and the rest among the first MFMAs of the next slice, so that the
    // workgroup's copies do not all enter the memory path at once.
    constexpr int NDEF = !VCE_DMA_DEFER        ? 0
                         : MODE == EPI_GRAD    ? VCE_DMA_DEFER_GRAD
                         : MODE == EPI_STORE   ? 0
                                               : VCE_DMA_DEFER_FWD;
    constexpr bool DEFER = NDEF > 0;
    constexpr int LH = LOADS - (NDEF < LOADS ? NDEF : LOADS);
    static_assert(!DEFER || 2 * (LOADS - LH) <= MA * NB, "deferred copies fit the first sub-step");
    auto issue_one = [&](auto kk, int kn, auto af) {
      constexpr int k = decltype(kk)::value;
      const int64_t kofs = static_cast<int64_t>(kn) * BK;
      const uint32_t stl = smem_lds + (kn % NS) * STAGE;
      const int64_t kleft = klen - kofs;
      if constexpr (k < SA::Q)
        sa.issue_q(k, stl, Ab + kofs * (AKM ? g.lda : 1) * ES, kleft, wave,
                   decltype(af)::value || sa.fast(kleft));
      else
        sb.issue_q(k - SA::Q, stl + A_BYTES, Bb + kofs * (BKM ? g.ldb : 1) * ES, kleft, wave,
                   decltype(af)::value || sb.fast(kleft));
    };
    auto kstep16 = [&](int kt, auto wait_all, auto issue_next, auto last, auto all_fast,
                       auto defer_in) {
      constexpr bool WAIT_ALL = decltype(wait_all)::value;
      constexpr bool ISSUE = decltype(issue_next)::value;
      constexpr bool LAST = decltype(last)::value;
      constexpr bool AF = decltype(all_fast)::value;
      constexpr bool DIN = DEFER && decltype(defer_in)::value;
      const char* st = smem + (kt % NS) * STAGE;
      auto none = [] {};
      auto nodma = [](auto) {};
      // the second half of slice kt+1's copies, when the previous step left it
      auto dma0 = [&](auto slot) {
        constexpr int s = decltype(slot)::value;
        if constexpr (DIN && s % 2 == 0 && s / 2 < LOADS - LH)  // every other MFMA
          issue_one(std::integral_constant<int, LH + s / 2>{}, kt + NS - 1, all_fast);
      };
      // first sub-step; its last groups read the second's first fragments
      sub16(st, 0, st, 1, std::true_type{}, none, dma0);
      if constexpr (!LAST) {
        const char* stn = smem + ((kt + 1) % NS) * STAGE;
        const char *pa = nullptr, *pb = nullptr;
        uint32_t stl = 0;
        int64_t kleft = 0;
        bool fast_a = true, fast_b = true;
        if constexpr (ISSUE) {
          const int kn = kt + NS;
          const int64_t kofs = static_cast<int64_t>(kn) * BK;
          stl = smem_lds + (kn % NS) * STAGE;
          kleft = klen - kofs;
          pa = Ab + kofs * (AKM ? g.lda : 1) * ES;
          pb = Bb + kofs * (BKM ? g.ldb : 1) * ES;
          fast_a = AF || sa.fast(kleft);
          fast_b = AF || sb.fast(kleft);
        }
        auto mid = [&] {
          // this wave's reads of slice kt are complete, its part of slice kt+1 is in
          __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
          if constexpr (WAIT_ALL)
            wait_vmcnt<0>();
          else
            wait_vmcnt<(NS - 2) * LOADS>();
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::"r"(smem) : "memory");
        };
        auto dma = [&](auto slot) {
          constexpr int k = decltype(slot)::value - (MA - 2) * NB;
          if constexpr (DEFER) {
            // load j before MFMA j * 2 NB / LH of the last two groups
            static_for<0, LH>([&](auto jj) {
              constexpr int j = decltype(jj)::value;
              if constexpr (ISSUE && k == j * 2 * NB / LH)
                issue_one(std::integral_constant<int, j>{}, kt + NS, all_fast);
            });
          } else if constexpr (ISSUE && k >= 0 && k < LOADS) {
            if constexpr (k < SA::Q)
              sa.issue_q(k, stl, pa, kleft, wave, fast_a);
            else
              sb.issue_q(k - SA::Q, stl + A_BYTES, pb, kleft, wave, fast_b);
          }
        };
        sub16(st, 1, stn, 0, std::true_type{}, mid, dma);
      } else {
        sub16(st, 1, st, 0, std::false_type{}, none, nodma);
      }
    };
    auto step = [&](int kt, auto wait_all, auto issue_next, auto last, auto all_fast,
                    auto defer_in) {
      if constexpr (M16)
        kstep16(kt, wait_all, issue_next, last, all_fast, defer_in);
      else
        kstep(kt, wait_all, issue_next, last, all_fast);
    };

    if (nk > 0) {
      // slice 0 in; queue slice NS-1; first fragments
      if (nk >= NS - 1)
        wait_vmcnt<(NS - 2) * LOADS>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::"r"(smem) : "memory");
      if (!SPREAD && NS - 1 < nk) issue(NS - 1);
      load_epi();
      asm volatile("" ::"r"(smem) : "memory");
      if constexpr (M16)
        read16(smem);
      else
        read_frags(smem, 0, fa[0], fb[0]);
      using F_ = std::false_type;
      using T_ = std::true_type;
      auto kloop = [&](auto af) {
        int kt = 0;
        if constexpr (SPREAD) {
          // kstep(kt) queues slice kt+NS-1; at its barrier the slices after
          // kt+1 that are in flight are kt+2 .. kt+NS-1
          for (; kt + NS - 1 < nk; ++kt) step(kt, F_{}, T_{}, F_{}, af, F_{});
          for (; kt + 1 < nk; ++kt) step(kt, T_{}, F_{}, F_{}, af, F_{});
          step(kt, T_{}, F_{}, T_{}, af, F_{});
        } else if constexpr (M16 && DEFER) {
          // two stages: a step after one that queued copies issues their
          // second half (slice 1 was queued whole before the loop)
          static_assert(NS == 2, "deferred copies assume two stages");
          if (kt + NS < nk) {
            step(kt, F_{}, T_{}, F_{}, af, F_{});
            for (++kt; kt + NS < nk; ++kt) step(kt, F_{}, T_{}, F_{}, af, T_{});
            if (kt + 1 < nk) {  // kt + NS == nk
              step(kt, F_{}, F_{}, F_{}, af, T_{});
              ++kt;
            }
          } else if (kt + 1 < nk) {  // nk == 2
            step(kt, F_{}, F_{}, F_{}, af, F_{});
            ++kt;
          }
          step(kt, T_{}, F_{}, T_{}, af, F_{});
        } else {
          for (; kt + NS < nk; ++kt) step(kt, F_{}, T_{}, F_{}, af, F_{});
          if (kt + NS == nk && kt + 1 < nk) {
            step(kt, F_{}, F_{}, F_{}, af, F_{});
            ++kt;
          }
          for (; kt + 1 < nk; ++kt) step(kt, T_{}, F_{}, F_{}, af, F_{});
          step(kt, T_{}, F_{}, T_{}, af, F_{});
        }
      };
#if VCE_KLOOP_SPLIT
      // whole tiles (the common case) run a K loop without per-load tests
      if (sa.fast(klen) && sb.fast(klen) && klen % BK == 0)
        kloop(std::true_type{});
      else
        kloop(std::false_type{});
#else
      kloop(std::false_type{});
#endif
    } else {
      load_epi();
    }
    // Every load of this tile has landed (the last K step waited for all of
    // them); saying so explicitly lets the epilogue use its inputs without a
    // wait that would also cover the next tile's prefetch.
    wait_vmcnt<0>();
    if constexpr (M16 && !E16) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
          rows32_layout(acc[i][j], acc16[2 * i][2 * j], acc16[2 * i][2 * j + 1],
                        acc16[2 * i + 1][2 * j], acc16[2 * i + 1][2 * j + 1]);
    }

    // every wave is done with the stage buffers: start the next tile's loads
    lds_barrier();
    const uint32_t Ln = L + per_xcd;
    const bool has_next = Ln < end;
    const TileGeom t = cur;
    if (has_next) {
      cur = decode_tile<BM, BN>(g, Ln);
      setup(cur);
      prologue();
    }

    // ---------------------------------------------------------------- epilogue
    // Outside the forward, the lane indices are taken afresh here, opaque to
    // the optimiser, so that nothing the epilogue derives from them is
    // computed at the top of the kernel and kept live (often in 64-bit form)
    // across the K loop (the forward's epilogue allocates better without).
    int lane_ep = lane;
    if constexpr (MODE != EPI_FWD) asm volatile("" : "+v"(lane_ep));
    {
    const int lane = lane_ep;
    const int half = lane >> 5, l32 = lane & 31;
    // Row of accumulator element r of block i (relative to the wave tile):
    //   i*32 + 8*(r/4) + 4*half + r%4 ;  its column: j*32 + l32.
    const int64_t vbase = t.m0 + wm * WM;

    if constexpr (E16 && MODE == EPI_FWD) {
      // 16x16 blocks: acc16[a][b] register r of lane l is wave-tile row
      // 16 a + 4 (l / 16) + r, column 16 b + l % 16; a token's 128 rows are
      // spread over the four lane groups l / 16, joined by two xor swaps
      const FwdArgs& f = e.fwd;
      const int grp = lane >> 4, c16 = lane & 15;
      const int lim = static_cast<int>(max(min(t.m_load - vbase, static_cast<int64_t>(WM)),
                                           static_cast<int64_t>(0)));
      const int lim_g = lim - 4 * grp;  // rows of this lane group: 16 a + r < lim_g
      if (lim != WM) {  // rows past the real vocabulary (or the shard) take no part
#pragma unroll
        for (int a = 0; a < MA; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * a + r >= lim_g) acc16[a][b][r] = -INFINITY;
      }
      float mj[NB], sj[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float m = -INFINITY;
#pragma unroll
        for (int a = 0; a < MA; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r) m = fmaxf(m, acc16[a][b][r]);
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        float sum = 0.0f;
        if (m != -INFINITY) {
          const float mb = m * kLog2e;
#pragma unroll
          for (int a = 0; a < MA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += fast_exp2(fmaf(acc16[a][b][r], kLog2e, -mb));
        }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        mj[b] = m;
        sj[b] = sum;
        const int col = wn * WN + 16 * b + c16;
        if (wm > 0 && grp == 0) red[(wm - 1) * BN + col] = make_float2(m, sum);

        // the owning tile stores the target logit (from the lane group holding its row)
        const int64_t dy = static_cast<int64_t>(yv[b]) - vbase;
        const bool mine = yv[b] >= 0 && dy >= 0 && dy < lim;
        if (__any(mine)) {
          const int loc = static_cast<int>(mine ? dy : 0);
          const int loc_g = loc - 4 * grp;
          float val = 0.0f;
#pragma unroll
          for (int a = 0; a < MA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) val = (16 * a + r == loc_g) ? acc16[a][b][r] : val;
          if (mine && ((loc >> 2) & 3) == grp) f.zt[t.n0 + col] = val;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (WAVES_M > 1) lds_barrier();
      // the first wave along M merges the pairs in wave order and stores them
      // (red is written again only after the next tile's K loop)
      if (wm == 0 && grp == 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int col = wn * WN + 16 * b + c16;
          float m = mj[b], sum = sj[b];
#pragma unroll
          for (int w = 1; w < WAVES_M; ++w) {
            const float2 o = red[(w - 1) * BN + col];
            lse_merge(m, sum, o.x, o.y);
          }
          const int64_t tt = t.n0 + col;
          if (tt < f.T) f.stats[t.tm * f.T + tt] = make_float2(m, sum);
        }
      }
    } else if constexpr (MODE == EPI_FWD) {
      const FwdArgs& f = e.fwd;
      // real rows of this wave's sub-tile: local rows [0, lim)  (m_load_end = V_real)
      const int lim = static_cast<int>(max(min(t.m_load - vbase, static_cast<int64_t>(WM)),
                                           static_cast<int64_t>(0)));
      const bool full = lim == WM;
      // Element r of block i sits at local row i*32 + 8*(r/4) + r%4 + 4*half;
      // comparisons move the lane's 4*half to the other side, so each is
      // against a compile-time constant.
      if (!full) {  // rows past the real vocabulary (or the shard) take no part
        const int lim_l = lim - 4 * half;
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (i * 32 + 8 * (r >> 2) + (r & 3) >= lim_l) acc[i][j][r] = -INFINITY;
      }
      float mj[NI], sj[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[i][j][r]);
        m = fmaxf(m, __shfl_xor(m, 32));
        float s = 0.0f;
        if (m != -INFINITY) {
          const float mb = m * kLog2e;
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += fast_exp2(fmaf(acc[i][j][r], kLog2e, -mb));
        }
        s += __shfl_xor(s, 32);
        mj[j] = m;
        sj[j] = s;
        const int col = wn * WN + j * 32 + l32;
        // waves past the first along M hand their pair to the first one
        if (wm > 0 && half == 0) red[(wm - 1) * BN + col] = make_float2(m, s);

        // the owning tile stores the target logit
        const int64_t dy = static_cast<int64_t>(yv[j]) - vbase;
        const bool mine = yv[j] >= 0 && dy >= 0 && dy < lim;
        if (__any(mine)) {
          const int loc = static_cast<int>(mine ? dy : 0);
          const int loc_l = loc - 4 * half;
          float val = 0.0f;
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              val = (i * 32 + 8 * (r >> 2) + (r & 3) == loc_l) ? acc[i][j][r] : val;
          if (mine && ((loc >> 2) & 1) == half) f.zt[t.n0 + col] = val;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (WAVES_M > 1) lds_barrier();
      // The first wave along M merges the pairs in wave order and stores them.
      // red is written again only after the next tile's K loop, whose barriers
      // every wave passes only after this merge, so no barrier follows.
      if (wm == 0 && half == 0) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int col = wn * WN + j * 32 + l32;
          float m = mj[j], s = sj[j];
#pragma unroll
          for (int w = 1; w < WAVES_M; ++w) {
            const float2 b = red[(w - 1) * BN + col];
            lse_merge(m, s, b.x, b.y);
          }
          const int64_t tt = t.n0 + col;
          if (tt < f.T) f.stats[t.tm * f.T + tt] = make_float2(m, s);
        }
      }
    } else if constexpr (MODE == EPI_ARGMAX) {
      const ArgArgs& a = e.arg;
      // real rows of this wave's sub-tile: local rows [0, lim)  (m_load_end = V_real)
      const int lim = static_cast<int>(max(min(t.m_load - vbase, static_cast<int64_t>(WM)),
                                           static_cast<int64_t>(0)));
      const int lim_l = lim - 4 * half;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        float bv = -INFINITY;
        int bi = -1;
        if (lim == WM) {
          // every row is real (the same for the whole wave): the largest value,
          // then the lowest of this lane's rows holding it (rows visited in
          // decreasing order, the last match kept)
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) bv = fmaxf(bv, acc[i][j][r]);
#pragma unroll
          for (int i = MI - 1; i >= 0; --i)
#pragma unroll
            for (int r = 15; r >= 0; --r)
              bi = (acc[i][j][r] == bv) ? i * 32 + 8 * (r >> 2) + (r & 3) + 4 * half : bi;
        } else {
          // this lane's rows in increasing order; strict > keeps the lowest row on ties
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int rl = i * 32 + 8 * (r >> 2) + (r & 3);  // row - 4*half
              const float v = acc[i][j][r];
              if (rl < lim_l && v > bv) {
                bv = v;
                bi = rl + 4 * half;
              }
            }
        }
        const float ov = __shfl_xor(bv, 32);
        const int oi = __shfl_xor(bi, 32);
        if (ov > bv || (ov == bv && oi >= 0 && (bi < 0 || oi < bi))) {
          bv = ov;
          bi = oi;
        }
        const int col = wn * WN + j * 32 + l32;
        const int tile_row = bi < 0 ? -1 : wm * WM + bi;
        if constexpr (WAVES_M > 1) {
          // every wave along M leaves its pair in LDS: nothing is held across the barrier
          if (half == 0) red[wm * BN + col] = make_float2(bv, __int_as_float(tile_row));
        } else if (half == 0) {
          const int64_t tt = t.n0 + col;
          if (tt < a.T) {
            a.val[t.tm * a.T + tt] = bv;
            a.idx[t.tm * a.T + tt] = tile_row < 0 ? -1 : static_cast<int32_t>(t.m0 + tile_row);
          }
        }
      }
      if constexpr (WAVES_M > 1) {
        lds_barrier();
        // the first wave along M merges in wave order (rows increase with the wave)
        if (wm == 0 && half == 0) {
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            const int col = wn * WN + j * 32 + l32;
            float bv = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int w = 0; w < WAVES_M; ++w) {
              const float2 o = red[w * BN + col];
              const int oi = __float_as_int(o.y);
              if (o.x > bv || (o.x == bv && oi >= 0 && (bi < 0 || oi < bi))) {
                bv = o.x;
                bi = oi;
              }
            }
            const int64_t tt = t.n0 + col;
            if (tt < a.T) {
              a.val[t.tm * a.T + tt] = bv;
              a.idx[t.tm * a.T + tt] = bi < 0 ? -1 : static_cast<int32_t>(t.m0 + bi);
            }
          }
        }
      }
    } else if constexpr (MODE == EPI_GRAD) {
      const GradArgs& gr = e.grad;
      // Element (i, 4q + c) of this lane sits at row vb + i*32 + 8*q + c of
      // the GEMM (vocabulary row v_off + that of the table). Limits and the
      // target are taken relative to vb and clamped to [-1, WM], so every
      // test is a 32-bit compare against a compile-time constant.
      const int64_t vb = vbase + 4 * half;
      auto rel = [&](int64_t x) {
        return static_cast<int>(max(min(x - vb, static_cast<int64_t>(WM)), static_cast<int64_t>(-1)));
      };
      const int real_l = rel(min(t.m_end, gr.V_real - gr.v_off));  // rows below are real classes
      const bool rows_real = real_l + 4 * half >= WM;  // the same for every lane of the wave
      const int end_l = rel(t.m_end);                                 // rows below exist
      E* Gp = static_cast<E*>(gr.G);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t tt = t.n0 + wn * WN + j * 32 + l32;
        const bool tin = tt < gr.T;
        const int64_t y = yv[j];
        const bool valid = tin && y >= 0 && y < gr.V_real;
        const int y_l = valid ? rel(y - gr.v_off) : -1;
        const int lim_l = valid ? real_l : -1;
        const float nl = lv[j] * kLog2e;
        const float sj = valid ? scale : 0.0f;
        E* grow = Gp + tt * gr.ldG + vb;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          float gv[16];
          if (rows_real) {
            // every row of the wave's tile is a real class: p <= 1 is finite,
            // and sj = 0 zeroes the rows of an ignored token
#pragma unroll
            for (int q = 0; q < 16; ++q)
              gv[q] = sj * fast_exp2(fmaf(acc[i][j][q], kLog2e, -nl));
            // the target row, if this block holds it for this lane (rare)
            if (static_cast<unsigned>(y_l - i * 32) < 32u) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (i * 32 + 8 * q + c == y_l) gv[4 * q + c] -= sj;
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                const int r = i * 32 + 8 * q + c;
                const float p = fast_exp2(fmaf(acc[i][j][4 * q + c], kLog2e, -nl));
                const float oh = (r == y_l) ? 1.0f : 0.0f;
                // select, never multiply, so a non-finite p of a discarded entry cannot leak
                gv[4 * q + c] = (r < lim_l) ? scale * (p - oh) : 0.0f;
              }
          }
          if constexpr (sizeof(E) == 2) {
            // the 32-row block lies inside the tile for both lanes of the pair
            if (gr.vec_store && tin && i * 32 + 32 <= end_l + 4 * half) {
              // lane pairs (l, l^32) trade quarter-blocks so that each lane
              // holds 8 consecutive rows twice: 16-byte stores. A half-swap
              // (v_permlane32_swap: lanes 32-63 of its first operand trade
              // places with lanes 0-31 of its second) of quarter-blocks 0 and
              // 1 leaves {0 of l, 0 of l^32} in the lower lanes and {1 of l^32,
              // 1 of l} in the upper ones: rows 8*half .. 8*half+7 of the
              // 16-row group in both; likewise 2 and 3.
              u32x2 P[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                P[q].x = pack_bf16x2(gv[4 * q], gv[4 * q + 1]);
                P[q].y = pack_bf16x2(gv[4 * q + 2], gv[4 * q + 3]);
              }
              const auto s0x = __builtin_amdgcn_permlane32_swap(P[0].x, P[1].x, false, false);
              const auto s0y = __builtin_amdgcn_permlane32_swap(P[0].y, P[1].y, false, false);
              const auto s1x = __builtin_amdgcn_permlane32_swap(P[2].x, P[3].x, false, false);
              const auto s1y = __builtin_amdgcn_permlane32_swap(P[2].y, P[3].y, false, false);
              const u32x4 p0 = {s0x[0], s0y[0], s0x[1], s0y[1]};
              const u32x4 p1 = {s1x[0], s1y[0], s1x[1], s1y[1]};
              E* base = Gp + tt * gr.ldG + vbase + i * 32 + 8 * half;
              *reinterpret_cast<u32x4*>(base) = p0;
              *reinterpret_cast<u32x4*>(base + 16) = p1;
            } else if (tin) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int r0 = i * 32 + 8 * q;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (r0 + c < end_l) grow[r0 + c] = f32_to_bf16(gv[4 * q + c]);
              }
            }
          } else {
            if (!tin) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int r0 = i * 32 + 8 * q;
              if (gr.vec_store && r0 + 3 < end_l) {
                f32x4 pk = {gv[4 * q], gv[4 * q + 1], gv[4 * q + 2], gv[4 * q + 3]};
                *reinterpret_cast<f32x4*>(grow + r0) = pk;
              } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                  if (r0 + c < end_l) grow[r0 + c] = gv[4 * q + c];
              }
            }
          }
        }
      }
    } else {  // EPI_STORE
      const StoreArgs& st = e.store;
      // split 0 writes (or adds into) C; every later K split writes (or adds
      // into, when an earlier launch left a sum there) its own partial
      // plane, which a fixed-order pass adds into C afterwards
      const bool first = t.ks == 0;
      float* Cp = first ? st.C : st.P + (t.ks - 1) * st.split_stride;
      const int64_t ldc = st.ldc;
      const bool accum = first ? st.accumulate != 0 : (t.ks - 1) < st.planes_held;
      // element (i, r) of this lane: row vb + i*32 + 8*(r/4) + r%4
      const int64_t vb = vbase + 4 * half;
      auto rel = [&](int64_t x) {
        return static_cast<int>(max(min(x - vb, static_cast<int64_t>(WM)), static_cast<int64_t>(-1)));
      };
      const int end_l = rel(t.m_end);
      const int zero_l = rel(st.m_zero_from);
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int64_t n = t.n0 + wn * WN + j * 32 + l32;
        if (n >= t.n_end) continue;
        float* col = Cp + vb * ldc + n;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = i * 32 + 8 * (r >> 2) + (r & 3);
            if (rr >= end_l) continue;
            const bool zero_row = rr >= zero_l;
            if (zero_row && accum) continue;
            float* dst = col + rr * ldc;
            const float v = zero_row ? 0.0f : acc[i][j][r];
            if (accum)  // the only writer of this element in this launch
              __hip_atomic_fetch_add(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
              *dst = v;
          }
      }
    }
    }

    if (!has_next) break;
    L = Ln;
  }
}

}  // namespace vce
